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
// every K/V tile staged in LDS serves 256 query rows.
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
// register staging), row-major with the 16-byte chunks of each row XOR-
// swizzled by a function of the row so that the reads below are free of
// bank conflicts.  K feeds the first product with 16-byte reads; V feeds
// the second through the gfx950 transposing read (ds_read_b64_tr_b16), which
// hands each lane four keys of one head dimension.
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
// maximum is used for the sum and for the output).
constexpr float RESCALE_LOG2 = 8.0f;

// LDS swizzles (16-byte chunk index XOR a function of the row), chosen so
// that the reads below hit distinct banks whether the LDS serves 128 or 256
// bytes per cycle.  K: 16 consecutive rows read one column chunk.  V: the
// transposing read takes 4 consecutive keys x 2-4 adjacent chunks.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  return D == 128 ? (row & 15) : ((row ^ (row >> 3)) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int key) {
  return D == 128 ? ((((key & 3) << 2) ^ ((key & 3) << 1)) & 14) : (2 * (key & 3));
}

template <int D, bool OF32>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2, 2))) void cowa_fwd_kernel(FwdParams p) {
  constexpr int CPR = D / 8;                  // 16-byte chunks per K/V row
  constexpr int TILE = BN * D;                // bf16 elements per K or V tile
  constexpr int LOADS = BN * CPR / 64 / NWAVES;  // direct loads per wave per tile
  static_assert(LOADS >= 1, "every wavefront loads part of each tile");
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
  int64_t qb = (int64_t)b * p.qs_b, kb = (int64_t)b * p.ks_b, vb = (int64_t)b * p.vs_b;
  int64_t ob = (int64_t)b * p.os_b, lse_base = ((int64_t)b * p.Hq + hq) * p.N;
  if (p.cu_seqlens) {
    const int start = p.cu_seqlens[b];
    N = min(p.cu_seqlens[b + 1] - start, p.N);
    if (qi * BM >= N) return;  // the whole workgroup: this tile is past the sequence
    qb = (int64_t)start * p.qs_t;
    kb = (int64_t)start * p.ks_t;
    vb = (int64_t)start * p.vs_t;
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
  const uint16_t* vbase = p.v + vb + (int64_t)h * p.vs_h;

  // Direct-load geometry: LDS chunk position P = (wave*LOADS + i)*64 + lane
  // holds row P / CPR, column chunk (P % CPR) ^ swizzle(row).  Per-lane
  // offsets inside a tile are fixed; the tile base is uniform.
  int ld_row[LOADS], ld_kcol[LOADS], ld_vcol[LOADS], ld_koff[LOADS], ld_voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int P = (wave * LOADS + i) * 64 + lane;
    ld_row[i] = P / CPR;
    ld_kcol[i] = ((P % CPR) ^ kswz<D>(ld_row[i])) * 8;
    ld_vcol[i] = ((P % CPR) ^ vswz<D>(ld_row[i])) * 8;
    ld_koff[i] = (int)(ld_row[i] * p.ks_t) + ld_kcol[i];
    ld_voff[i] = (int)(ld_row[i] * p.vs_t) + ld_vcol[i];
  }
  // Loads of one K (or V) tile into LDS buffer dst.  Keys past N (ragged last
  // tile) are clamped to N - 1: they only occur in tiles the plan marks
  // partial, where they are masked (probability exactly 0).
  auto load_tile = [&](const uint16_t* base, int64_t stride, const int* off, const int* col,
                       int kj, uint16_t* dst) {
    const int key0 = kj * BN;
    if (key0 + BN <= N) {
      const uint16_t* t = base + (int64_t)key0 * stride;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) g2lds16(t + off[i], dst + (wave * LOADS + i) * 512);
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        int key = key0 + ld_row[i];
        key = key < N ? key : N - 1;
        g2lds16(base + (int64_t)key * stride + col[i], dst + (wave * LOADS + i) * 512);
      }
    }
  };

  // K read offsets (first product, A operand): row 32*blk + l32, chunk 2*ks + hl
  int k_off[2][NK];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      k_off[blk][ks] = (32 * blk + l32) * D + (((2 * ks + hl) ^ kswz<D>(32 * blk + l32)) * 8);
  // V transposed-read offsets (second product, A operand): for 16-key step st,
  // d block db and half ri, lane reads key 16*st + 8*ri + 4*hl + (lane&15)/4 at
  // dims 32*db + 16*((lane>>4)&1) + 4*(lane&3) .. +3.
  const int r16 = lane & 15;
  const int gi = (lane >> 4) & 1;
  int v_off[2][ND];
#pragma unroll
  for (int ri = 0; ri < 2; ++ri)
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int key = 8 * ri + 4 * hl + (r16 >> 2);
      const int d = 32 * db + 16 * gi + 4 * (r16 & 3);
      v_off[ri][db] = key * D + (((d >> 3) ^ vswz<D>(key)) * 8) + (d & 7);
    }

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

  // S^T = K Q^T for the 64 keys of the K tile in buffer kb
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

  // Pipeline: iteration e holds S(e) in registers, reads K(e+1) and V(e) from
  // LDS, and streams K(e+2) and V(e+1) into the buffers freed last iteration.
  // The MFMAs of S(e+1) are independent of the softmax of S(e), so they
  // overlap it.
  f32x16 s_first[2];
  int c_cur = 0, c_n1 = 0;  // plan entries of tiles e and e + 1
  if (e0 < e1) {
    c_cur = entry(e0);
    c_n1 = e0 + 1 < e1 ? entry(e0 + 1) : 0;
    load_tile(kbase, p.ks_t, ld_koff, ld_kcol, c_cur & 0x7fffffff, K0);
    load_tile(vbase, p.vs_t, ld_voff, ld_vcol, c_cur & 0x7fffffff, V0);
    if (e0 + 1 < e1) load_tile(kbase, p.ks_t, ld_koff, ld_kcol, c_n1 & 0x7fffffff, K1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    qk(K0, s_first);
    // every wave has read K(e0) before its buffer is refilled
    __syncthreads();
  }

  // One pipeline step for tile e; s_cur holds S(e), s_nxt receives S(e+1).
  // Reads K(e+1) from Kr and V(e) from Vr; K(e+2) streams into Kw, V(e+1) into Vw.
  auto step = [&](int e, f32x16* s_cur, f32x16* s_nxt, const uint16_t* Kr, const uint16_t* Vr,
                  uint16_t* Kw, uint16_t* Vw) {
    const int kj = c_cur & 0x7fffffff;
    const bool full = c_cur < 0;
    const bool has_next = e + 1 < e1;
    // plan entry of tile e + 2 (the chunk moves on when e + 2 leaves it)
    int c_n2 = 0;
    if (e + 2 < e1) {
      if (e + 2 - pbase == 64) {
        pbase += 64;
        pchunk = plan_chunk(pbase);
      }
      c_n2 = entry(e + 2);
      load_tile(kbase, p.ks_t, ld_koff, ld_kcol, c_n2 & 0x7fffffff, Kw);
    }
    if (has_next) load_tile(vbase, p.vs_t, ld_voff, ld_vcol, c_n1 & 0x7fffffff, Vw);

    if (!full) {
      // register i of block blk holds key kj*64 + 4 hl + o
      const uint64_t vis = row_visible_bits(hp, q_row, kj * BN + 4 * hl);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s_cur[blk][i] = keep_if(s_cur[blk][i], vis, 32 * blk + 8 * (i >> 2) + (i & 3));
    }

    float mt = NEG_INF;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s_cur[blk][i]);
    mt = pair_max(mt);
    // raise the reference maximum only where it grew past the threshold
    // (always on a row's first visible key: m_run = -inf gives +inf)
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

    // ---- one basic block: S(e+1) MFMAs, softmax of S(e), P.V MFMAs ----
    // (unconditional so that the scheduler can interleave it with the
    // softmax; on a row's last tile it reads a stale buffer and is unused)
    qk(Kr, s_nxt);
    unsigned pk[2][8];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[blk][2 * i], p.scale_log2, -mb));
        const float c = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[blk][2 * i + 1], p.scale_log2, -mb));
        pk[blk][i] = pack_bf16(a, c);
        l_run += a + c;
      }
    const uint16_t* Vs = Vr;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int blk = st >> 1;
      const int o4 = (st & 1) * 4;
      const u32x4 pw = {pk[blk][o4], pk[blk][o4 + 1], pk[blk][o4 + 2], pk[blk][o4 + 3]};
      const bf16x8 bv = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const i16x4 lo = lds_read_tr(Vs + st * 16 * D + v_off[0][db]);
        const i16x4 hi = lds_read_tr(Vs + st * 16 * D + v_off[1][db]);
        const i16x4 a8[2] = {lo, hi};
        const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[db], 0, 0, 0);
      }
    }
    // interleave: MFMAs of S(e+1) with the softmax VALU of S(e), then the
    // P.V MFMAs with their transposed V reads
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    c_cur = c_n1;
    c_n1 = c_n2;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // unrolled by two so the two S register sets and the buffers alternate
  // without copies or run-time buffer selection
  f32x16 s_alt[2];
  for (int e = e0; e < e1; e += 2) {
    step(e, s_first, s_alt, K1, V0, K0, V1);
    if (e + 1 < e1) step(e + 1, s_alt, s_first, K0, V1, K1, V0);
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
