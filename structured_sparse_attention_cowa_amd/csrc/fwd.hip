// CoWA prefill forward for gfx950 (CDNA4): bf16 MFMA, LDS-staged K/V tiles,
// fp32 online softmax, driven by the visible-tile lists of cowa_plan.
//
// What is computed ("CoWindow Attention: Full Causal Coverage Is a
// Collective Property", Abstract; "Splitting long-range windows across KV
// heads beats duplicating them at lower cost", mechanism paragraph and the
// paragraph on what CoWA does not claim): for every query head, a softmax over
// that head's own visible keys (shared sink, shared local window, the band of
// its global KV head).  Only the key tiles the plan lists are loaded; only
// tiles the plan marks partial are masked.
//
// Workgroup = 8 wavefronts = 256 query rows of one (batch, query head), so
// every K/V tile staged in LDS serves 256 query rows.  Wavefront w runs on
// SIMD w % 4, so each SIMD holds one wavefront of waves 0-3 (group A) and one
// of waves 4-7 (group B); the two groups run the pipeline half a step apart
// (below), so that on every SIMD one of them issues MFMAs while the other
// runs its softmax.
// Each wavefront owns 32 query rows and works in the transposed frame:
//   S^T (32 keys x 32 queries) = K (32 x d) . Q^T (d x 32)     [MFMA 32x32x16]
//   O^T (d x 32 queries)      += V^T (d x 64) . P^T (64 x 32)   [MFMA 32x32x16]
// so every lane owns one query column: its softmax statistics are per-lane
// scalars, the row max needs one exchange with the lane 32 away, and the
// accumulator rescale is a per-lane scalar multiply.  The P^T operand of the
// second product is the first product's accumulator, converted to bf16 in
// place; the key order inside each 16-key step follows the accumulator
// layout (lane half 0 holds keys 0-3 and 8-11, half 1 keys 4-7 and 12-15).
//
// K and V tiles go from HBM straight into LDS (16 bytes per lane, no
// register staging), with the 16-byte chunks of each row XOR-swizzled by a
// function of the row so that the reads below are free of bank conflicts.
// K tiles are row-major (key rows) and feed the first product with 16-byte
// reads.  V is read from a head-dim-major copy that a transpose kernel writes
// into the workspace first (one row per head dim, the keys of each 16-key
// group in the order the P^T operand takes them), so each operand of the
// second product is also one 16-byte read: the LDS serves the transposing
// read (ds_read_b64_tr_b16) that the row-major V would need at well under
// half the rate of 16-byte reads.
#include <hip/hip_runtime.h>

#include "cowa_internal.h"
#include "kernel_util.h"

namespace cowa {
namespace {

using namespace kern;

constexpr int BM = kFwdBlockM;  // query rows per workgroup (32 per wavefront)
constexpr int BN = kFwdBlockN;  // 64 keys per tile
constexpr int NWAVES = BM / 32;
constexpr int NTHREADS = 64 * NWAVES;

// The running maximum is only raised when a row's maximum grows by more than
// 2^RESCALE_LOG2 in probability terms; until then the stale maximum is kept
// and probabilities may reach 2^RESCALE_LOG2 (exact: the same reference
// maximum is used for the sum and for the output).  At 2^16 the sums stay far
// inside fp32 range (at most 2^16 per key) and bf16 keeps its relative
// precision, while a row's reference is rarely raised after its first tile,
// even with a few large-norm keys.
constexpr float RESCALE_LOG2 = 16.0f;
constexpr float RESCALE_BOUND = 65536.0f;  // 2^RESCALE_LOG2

// K-tile swizzle (16-byte chunk index XOR a function of the row), chosen so
// that 16 consecutive rows reading one column chunk hit distinct banks
// whether the LDS serves 128 or 256 bytes per cycle.  (V tiles use swz_tr8.)
template <int D>
__device__ __forceinline__ int kswz(int row) {
  return D == 128 ? (row & 15) : ((row ^ (row >> 3)) & 7);
}

// V head-dim-major into the workspace: grid (npad / 64, H_kv, B), one
// workgroup per 64 keys of one (sequence, KV head), through LDS.  Keys past
// the sequence's end are written as zeros (a plan built for the longest
// sequence may list such tiles: their keys are masked, and a zero value keeps
// the masked products exactly zero).
template <int D>
__global__ __launch_bounds__(256) void cowa_fwd_vt_kernel(FwdParams p) {
  constexpr int CH = D / 8;  // 16-byte chunks per key row
  __shared__ __attribute__((aligned(16))) uint16_t tile[BN][D + 8];
  const int tid = threadIdx.x;
  const int k0 = blockIdx.x * BN;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  int n = p.N;
  int64_t base = (int64_t)b * p.vs_b + (int64_t)h * p.vs_h;
  if (p.cu_seqlens) {
    const int start = p.cu_seqlens[b];
    n = min(p.cu_seqlens[b + 1] - start, p.N);
    base = (int64_t)start * p.vs_t + (int64_t)h * p.vs_h;
  }
  for (int c = tid; c < BN * CH; c += 256) {
    const int r = c / CH, k = c % CH;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (k0 + r < n) w = ldg16(p.v + base + (int64_t)(k0 + r) * p.vs_t + 8 * k);
    *reinterpret_cast<u32x4*>(&tile[r][8 * k]) = w;
  }
  __syncthreads();
  // row dd of the copy: 8 chunks of 8 positions, position q holding key
  // k0 + tr16_position(q)
  uint16_t* dst = p.vt + ((int64_t)b * p.Hkv + h) * D * p.npad + k0;
  for (int c = tid; c < D * 8; c += 256) {
    const int dd = c >> 3, k = c & 7;
    unsigned w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q0 = 8 * k + 2 * j;
      w[j] = (unsigned)tile[tr16_position(q0)][dd] |
             ((unsigned)tile[tr16_position(q0 + 1)][dd] << 16);
    }
    *reinterpret_cast<u32x4*>(dst + (int64_t)dd * p.npad + 8 * k) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

template <int D, bool OF32>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2, 2))) void cowa_fwd_kernel(FwdParams p) {
  constexpr int CPR = D / 8;                  // 16-byte chunks per K/V row
  constexpr int TILE = BN * D;                // bf16 elements per K or V tile
  constexpr int ND = D / 32;                  // 32-wide d blocks of O^T
  constexpr int NK = D / 16;                  // 16-deep k steps of Q.K

  // One LDS variable per tile buffer: the compiler tells distinct variables
  // apart, so the loads streaming into one buffer stay in flight while the
  // step reads another (within one variable it would wait for them first).
  __shared__ __attribute__((aligned(16))) uint16_t K0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t K1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  // Heavy-first order over the whole batch (later query tiles see more keys),
  // dealt to the XCDs in chunks.  The dispatcher sends workgroup i to XCD
  // i mod 8; chunk c of xcd_chunk consecutive logical workgroups (a few query
  // tiles with all their heads, which read the same K/V tiles) goes to XCD
  // c mod 8, so those reads share one L2.  Padding workgroups exit at once.
  const int per_qi = p.B * p.Hq;
  const int wg = xcd_logical(blockIdx.x, p.xcd_chunk, per_qi * p.nqt);
  if (wg < 0) return;
  const int qi = p.nqt - 1 - wg / per_qi;
  const int rem = wg - (wg / per_qi) * per_qi;
  const int b = rem / p.Hq;
  const int hq = rem - b * p.Hq;
  const int h = hq / p.G;

  // this sequence's length and the offsets of its rows
  int N = p.N;
  int64_t qb = (int64_t)b * p.qs_b, kb = (int64_t)b * p.ks_b;
  int64_t ob = (int64_t)b * p.os_b, lse_base = ((int64_t)b * p.Hq + hq) * p.N;
  if (p.cu_seqlens) {
    const int start = p.cu_seqlens[b];
    N = min(p.cu_seqlens[b + 1] - start, p.N);
    if (qi * BM >= N) return;  // the whole workgroup: this tile is past the sequence
    qb = (int64_t)start * p.qs_t;
    kb = (int64_t)start * p.ks_t;
    ob = (int64_t)start * p.os_t;
    lse_base = (int64_t)hq * p.total_tokens + start;
  }
  const HeadPattern hp = head_pattern(p.sink, p.window, p.band,
                                      band_slot(p.kv_head_offset + h, p.n_bands), p.causal);

  const int q_row = qi * BM + wave * 32 + l32;
  const int q_row_c = q_row < N ? q_row : N - 1;

  bf16x8 qf[NK];
  {
    const uint16_t* qp = p.q + qb + (int64_t)q_row_c * p.qs_t + (int64_t)hq * p.qs_h;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, ldg16(qp + 16 * ks + 8 * hl));
    // complete before the tile loop, which then starts with no register load
    // in flight (otherwise it waits for its own prefetch)
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) asm volatile("" : : "v"(qf[ks]));
  }

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};
  float m_run = NEG_INF;
  float l_run = 0.f;

  const int row = h * p.nqt + qi;
  const int e0 = p.row_ptr[row];
  const int e1 = p.row_ptr[row + 1];
  const uint16_t* kbase = p.k + kb + (int64_t)h * p.ks_h;
  // V: the head-dim-major copy (rows d of npad keys) of this sequence and head
  const uint16_t* vbase = p.vt + ((int64_t)b * p.Hkv + h) * D * p.npad;

  // Group A streams whole tiles: LDS chunk position P = (wave * LOADS_A + i)
  // * 64 + lane of a K tile holds row P / CPR, column chunk (P % CPR) ^
  // kswz(row); of a V tile, row hdm_load_row(P), chunk hdm_load_chunk(P).
  // Keys past N (ragged last tile) are clamped to N - 1: they only occur in
  // tiles the plan marks partial, where they are masked (probability exactly
  // 0).  The loads are buffer loads to LDS (buffer_load ... lds) through a
  // resource based at the tile: with the global form of the direct-to-LDS
  // load the compiler waits for every outstanding LDS read at each one.
  // Byte offsets inside a tile stay below 2^31 (checked on the host).
  constexpr int HALF = NWAVES / 2;
  constexpr int LOADS_A = BN * CPR / 64 / HALF;   // K tile loads per group-A lane
  constexpr int VLOADS_A = D * 8 / 64 / HALF;     // V tile loads per group-A lane
  static_assert(LOADS_A >= 1 && VLOADS_A >= 1, "group A loads whole tiles");
  const bool grpB = wave >= HALF;
  const int wa = grpB ? 0 : wave;
  auto ld_row = [&](int i) { return ((wa * LOADS_A + i) * 64 + lane) / CPR; };
  auto ld_col = [&](int i) { return ((lane % CPR) ^ kswz<D>(ld_row(i))) * 8; };
  int ld_koff[LOADS_A];
#pragma unroll
  for (int i = 0; i < LOADS_A; ++i) ld_koff[i] = (int)(ld_row(i) * p.ks_t) + ld_col(i);
  int ld_voff[VLOADS_A];
#pragma unroll
  for (int i = 0; i < VLOADS_A; ++i) {
    const int P = (wa * VLOADS_A + i) * 64 + lane;
    ld_voff[i] = hdm_load_row(P) * p.npad + hdm_load_chunk(P) * 8;
  }
  auto load_k = [&](const uint16_t* base, int64_t stride, const int* off, int kj,
                    uint16_t* dst) {
    const int key0 = kj * BN;
    const __amdgpu_buffer_rsrc_t rs = lds_rsrc(base + (int64_t)key0 * stride);
    if (key0 + BN <= N) {
#pragma unroll
      for (int i = 0; i < LOADS_A; ++i) buf2lds16(rs, off[i] * 2, dst + (wa * LOADS_A + i) * 512);
    } else {
#pragma unroll
      for (int i = 0; i < LOADS_A; ++i) {
        int key = key0 + ld_row(i);
        key = key < N ? key : N - 1;
        buf2lds16(rs, (int)(((int64_t)(key - key0) * stride + ld_col(i)) * 2),
                  dst + (wa * LOADS_A + i) * 512);
      }
    }
  };
  auto load_v = [&](int kj, uint16_t* dst) {
    const __amdgpu_buffer_rsrc_t rs = lds_rsrc(vbase + (int64_t)kj * BN);
#pragma unroll
    for (int i = 0; i < VLOADS_A; ++i)
      buf2lds16(rs, ld_voff[i] * 2, dst + (wa * VLOADS_A + i) * 512);
  };

  // K read offsets (first product, A operand): row 32*blk + l32, chunk 2*ks + hl.
  // At d = 128 the swizzle repeats every 16 rows, so block 1 reads 32 rows
  // (a constant) further and only block 0's offsets occupy registers.
  int k_off[2][NK];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      k_off[blk][ks] = (blk == 1 && D == 128)
                           ? k_off[0][ks] + 32 * D
                           : (32 * blk + l32) * D + (((2 * ks + hl) ^ kswz<D>(32 * blk + l32)) * 8);
  // V read offsets (second product, A operand): for 16-key step st and d
  // block db the lane reads row 32*db + l32, chunk 2*st + hl, i.e. the 8 keys
  // (in the copy's order) that its P operand holds
  static_assert(BN == 64, "head-dim-major tiles hold 64 keys per row");
  int v_off[ND][4];
  hdm_read_offsets<D>(lane, v_off);

  // Plan entries travel 64 at a time, one per lane (tile index with the
  // full-tile flag in bit 31), and are picked out with readlane.
  auto plan_chunk = [&](int base) {
    const int e = base + lane;
    return e < e1 ? (p.col[e] | (p.flags[e] ? (int)0x80000000 : 0)) : 0;
  };
  int pbase = e0;
  int pchunk = plan_chunk(pbase);
  auto entry = [&](int e) {  // requires pbase <= e < pbase + 64
    return __builtin_amdgcn_readlane(pchunk, e - pbase);
  };

  // S^T = K Q^T for the 64 keys of the K tile in buffer Ks
  auto qk = [&](const uint16_t* Ks, f32x16* s) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + k_off[blk][ks]);
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[blk], 0, 0, 0);
      }
    }
  };

  // Every wave runs the same sequence of half-steps, M(e0-1), V(e0), M(e0),
  // V(e0+1), ..., M(e1-1), separated by workgroup barriers: M(e-1) computes
  // S(e) = K(e) Q^T and O^T += V(e-1)^T P(e-1) (MFMA work), V(e) masks S(e),
  // updates the row statistics and makes P(e) (VALU work).  Group B runs one
  // half-step behind group A (one extra barrier before its loop, A one after
  // its last product), so on every SIMD one wave issues MFMAs while the other
  // runs the softmax.  Tile e sits in buffers e mod 2 (relative to e0); group
  // A's M(e-1) streams K(e+1) and V(e) into the buffers both groups finished
  // reading two half-steps before, and the barrier after V(e) waits for them.
  f32x16 s[2];
  unsigned pk[2][8];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int i = 0; i < 8; ++i) pk[blk][i] = 0u;
  int c_cur = 0;  // plan entry of tile e
  if (e0 < e1) {
    c_cur = entry(e0);
    if (!grpB) load_k(kbase, p.ks_t, ld_koff, c_cur & 0x7fffffff, K0);
    // V1 starts as zeros: M(e0-1) multiplies it by P = 0
    for (int i = tid; i < TILE / 8; i += NTHREADS)
      *reinterpret_cast<u32x4*>(V1 + 8 * i) = u32x4{0u, 0u, 0u, 0u};
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (grpB) __builtin_amdgcn_s_barrier();
  }

  auto valu_half = [&](int c) {
    const int kj = c & 0x7fffffff;
    const bool full = c < 0;
    if (__builtin_expect(!full, 0)) {
      const uint64_t vis = row_visible_bits(hp, q_row, kj * BN + 4 * hl);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[blk][i] = keep_if(s[blk][i], vis, 32 * blk + 8 * (i >> 2) + (i & 3));
    }
    // Probabilities against the current reference maximum first.  If each
    // lane's sum (which bounds every one of its terms) stays at or below
    // 2^RESCALE_LOG2, no key of the row exceeds the reference by more than
    // the threshold, the reference stays, and the row maximum is not needed.
    // Otherwise, and on a row's first step (no reference yet), the wavefront
    // takes the maximum, raises the reference where it grew, and makes the
    // probabilities again.
    float lp = 0.f;
    {
      const float mb = m_run * p.scale_log2;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][2 * i], p.scale_log2, -mb));
          const float c2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][2 * i + 1], p.scale_log2, -mb));
          pk[blk][i] = pack_bf16(a, c2);
          lp += a + c2;
        }
    }
    const bool slow = !(lp <= RESCALE_BOUND) || m_run == NEG_INF;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(slow) != 0, 0)) {
      float mt = NEG_INF;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[blk][i]);
      mt = pair_max(mt);
      const bool grow = (mt - m_run) * p.scale_log2 > RESCALE_LOG2;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mt : m_run;
        const float alpha =
            m_run == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * p.scale_log2);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < ND; ++i) acc[i] *= alpha;
      }
      const float mb = m_run == NEG_INF ? 0.f : m_run * p.scale_log2;
      lp = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][2 * i], p.scale_log2, -mb));
          const float c2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][2 * i + 1], p.scale_log2, -mb));
          pk[blk][i] = pack_bf16(a, c2);
          lp += a + c2;
        }
    }
    l_run += lp;
    // P is made in this half: the compiler may not sink this arithmetic past
    // the barrier into the MFMA half that consumes it
    asm volatile("" : "+v"(pk[0][0]), "+v"(pk[0][1]), "+v"(pk[0][2]), "+v"(pk[0][3]),
                 "+v"(pk[0][4]), "+v"(pk[0][5]), "+v"(pk[0][6]), "+v"(pk[0][7]));
    asm volatile("" : "+v"(pk[1][0]), "+v"(pk[1][1]), "+v"(pk[1][2]), "+v"(pk[1][3]),
                 "+v"(pk[1][4]), "+v"(pk[1][5]), "+v"(pk[1][6]), "+v"(pk[1][7]));
  };
  auto pv = [&](const uint16_t* Vr) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int blk = st >> 1;
      const int o4 = (st & 1) * 4;
      const u32x4 pw = {pk[blk][o4], pk[blk][o4 + 1], pk[blk][o4 + 2], pk[blk][o4 + 3]};
      const bf16x8 bv = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vr + v_off[db][st]);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[db], 0, 0, 0);
      }
    }
  };
  // iteration e: K(e) in Kc, V(e-1) in Vp; group A streams K(e+1) into Kn
  // and V(e) into Vc
  auto iter = [&](int e, const uint16_t* Kc, uint16_t* Kn, uint16_t* Vc, const uint16_t* Vp) {
    int c_n1 = 0;
    if (e + 1 < e1) {
      if (e + 1 - pbase == 64) {
        pbase += 64;
        pchunk = plan_chunk(pbase);
      }
      c_n1 = entry(e + 1);
    }
    if (!grpB) {
      if (e + 1 < e1) load_k(kbase, p.ks_t, ld_koff, c_n1 & 0x7fffffff, Kn);
      load_v(c_cur & 0x7fffffff, Vc);
    }
    // M(e-1): 32 MFMAs, each fed by one 16-byte LDS read issued six reads
    // ahead
    qk(Kc, s);
    pv(Vp);
#pragma unroll
    for (int i = 0; i < 6; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // S is complete in this half (not sunk into the VALU half that reads it)
    asm volatile("" : "+v"(s[0]), "+v"(s[1]));
    // Every LDS read of this half is issued before the barrier: group A's
    // next loads overwrite Vp after it.  (No wait here: group A's tile loads
    // stay in flight across this barrier.)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    // V(e)
    valu_half(c_cur);
    c_cur = c_n1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int e = e0; e < e1; e += 2) {
    iter(e, K0, K1, V0, V1);
    if (e + 1 < e1) iter(e + 1, K1, K0, V1, V0);
  }
  // M(e1-1): the last tile's P.V product (no further tile)
  if (e0 < e1) {
    pv(((e1 - 1 - e0) & 1) ? V1 : V0);
    if (!grpB) __builtin_amdgcn_s_barrier();
  }

  const float l_tot = pair_sum(l_run);
  if (q_row < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    char* obase = reinterpret_cast<char*>(p.o);
    const int64_t oidx = ob + (int64_t)q_row * p.os_t + (int64_t)hq * p.os_h;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int gi2 = 0; gi2 < 4; ++gi2) {
        const int dd = 32 * db + 8 * gi2 + 4 * hl;
        const float v0 = acc[db][4 * gi2 + 0] * inv, v1 = acc[db][4 * gi2 + 1] * inv;
        const float v2 = acc[db][4 * gi2 + 2] * inv, v3 = acc[db][4 * gi2 + 3] * inv;
        if (OF32) {
          *reinterpret_cast<f32x4*>(obase + (oidx + dd) * 4) = f32x4{v0, v1, v2, v3};
        } else {
          *reinterpret_cast<u32x2*>(obase + (oidx + dd) * 2) =
              u32x2{pack_bf16(v0, v1), pack_bf16(v2, v3)};
        }
      }
    if (hl == 0) {
      const float lse = l_tot > 0.f ? m_run * p.scale + __logf(l_tot) : NEG_INF;
      p.lse[lse_base + q_row] = lse;
    }
  }
}

}  // namespace

int launch_fwd(const FwdParams& p_in, int d, int o_f32, void* stream) {
  // default chunk (packed sequences): whole query tiles with all their
  // (sequence, head) pairs, up to 8 of them
  FwdParams p = p_in;
  const int64_t per_qi = (int64_t)p.B * p.Hq;
  if (p.xcd_chunk <= 0) p.xcd_chunk = xcd_chunk(per_qi, p.nqt, 8);
  const dim3 grid((unsigned)xcd_grid(per_qi * p.nqt, p.xcd_chunk));
  const dim3 block(NTHREADS);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 vt_grid((unsigned)(p.npad / BN), (unsigned)p.Hkv, (unsigned)p.B);
  if (d == 128)
    hipLaunchKernelGGL(cowa_fwd_vt_kernel<128>, vt_grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(cowa_fwd_vt_kernel<64>, vt_grid, dim3(256), 0, s, p);
  if (d == 128) {
    if (o_f32)
      hipLaunchKernelGGL((cowa_fwd_kernel<128, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((cowa_fwd_kernel<128, false>), grid, block, 0, s, p);
  } else {
    if (o_f32)
      hipLaunchKernelGGL((cowa_fwd_kernel<64, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((cowa_fwd_kernel<64, false>), grid, block, 0, s, p);
  }
  return (int)hipGetLastError();
}

}  // namespace cowa
