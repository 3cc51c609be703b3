// CoWA prefill backward for gfx950 (CDNA4): dQ, dK, dV on the visible tiles
// only, bf16 MFMA with fp32 accumulation.
//
// What is differentiated ("CoWindow Attention: Full Causal Coverage Is a
// Collective Property", Abstract, training latency of the operator): for
// each query head, O_t = sum_j P_tj v_j with P_tj = exp(scale q_t.k_j - LSE_t)
// over that head's visible keys (sink, local window, its global KV head's
// band).  With D_t = dO_t . O_t and dS_tj = P_tj (dO_t . v_j - D_t):
//   dQ_t = scale sum_j dS_tj k_j
//   dK_j = scale sum_{t, heads of the group} dS_tj q_t
//   dV_j = sum_{t, heads of the group} P_tj dO_t
// P is recomputed from the forward's LSE, so no probability matrix is stored.
//
// Four kernels on the caller's stream:
//   delta  D_t and LSE in base-2 units into the workspace (rows padded to a
//          multiple of 64; padding rows get LSE = +inf, so P = 0 there);
//   dQ     one workgroup per (batch, query head, 256-row query tile), the
//          forward's query-major plan.  Each wavefront owns 32 query rows in
//          the transposed frame of the forward: S^T = K Q^T and dP^T = V dO^T
//          (lane = query column, so LSE and D are per-lane scalars), then
//          dQ^T += K^T dS^T with K read through the transposing LDS read;
//   dK/dV  one workgroup per (batch, KV head, 128-key tile), the key-major
//          plan.  Each wavefront owns 32 keys whose K and V rows stay in
//          registers; for every query head of the group and every visible
//          64-row query tile: S = Q K^T, dP = dO V^T (lane = key column), then
//          dV^T += dO^T P and dK^T += Q^T dS with dO and Q read transposed.
//          Summing the group's query heads inside the workgroup needs no
//          atomics.  Key tiles holding sink keys are seen by every query
//          tile; their step lists are cut into parts that run as separate
//          workgroups writing fp32 partials, which a last kernel sums in a
//          fixed order (the fourth kernel), so the result stays deterministic.
// Tiles stream from HBM straight into LDS (16 bytes per lane), double
// buffered, with one swizzle that serves both the plain and the transposing
// reads without bank conflicts.
#include <hip/hip_runtime.h>

#include "cowa_internal.h"
#include "kernel_util.h"

// key tiles per XCD chunk of the dK/dV grid (the dQ grid takes up to 8 query
// tiles): with 8, the K/V and Q/dO re-reads of neighbouring tiles mostly hit
// the XCD's L2 (32 was slower, from L2 thrash across the chunk's span)
constexpr int KV_CHUNK_TILES = 8;

namespace cowa {
namespace {

using namespace kern;

// Every kernel takes the head dimension D (64 or 128) as a template argument;
// with it, CPR = D / 8 16-byte chunks per row, NK = D / 16 16-deep k steps
// over the head dimension and ND = D / 32 32-wide head-dimension blocks of an
// accumulator.

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Sequence b: its first token row and its length.  Packed sequences take
// both from cu_seqlens (the b strides are 0); the batched layout has row 0
// and length N (its b strides select the sequence).  A negative length is an
// empty sequence.
struct SeqSpan {
  int start, n;
};
__device__ __forceinline__ SeqSpan seq_span(const BwdParams& p, int b) {
  if (!p.cu_seqlens) return {0, p.N};
  const int s = p.cu_seqlens[b];
  return {s, min(p.cu_seqlens[b + 1] - s, p.N)};
}

// ---------------------------------------------------------------- delta --
constexpr int DELTA_ROWS = 16;  // 16 lanes per row, 8 head dims each (lanes past D idle)

template <int D>
__global__ __launch_bounds__(256) void cowa_bwd_delta_kernel(BwdParams p) {
  const int tid = threadIdx.x;
  const int sub = tid & 15;
  const int t = blockIdx.x * DELTA_ROWS + (tid >> 4);
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const SeqSpan sp = seq_span(p, b);
  const int64_t row = (int64_t)sp.start + t;  // token row of position t
  float acc = 0.f;
  if (t < sp.n && 8 * sub < D) {
    const u32x4 dw = ldg16(p.dout + (int64_t)b * p.dos_b + row * p.dos_t +
                           (int64_t)hq * p.dos_h + 8 * sub);
    const int64_t oi = (int64_t)b * p.os_b + row * p.os_t + (int64_t)hq * p.os_h + 8 * sub;
    float o[8];
    if (p.o_f32) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.o) + oi);
      const f32x4 c = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.o) + oi + 4);
      for (int e = 0; e < 4; ++e) {
        o[e] = a[e];
        o[4 + e] = c[e];
      }
    } else {
      const u32x4 ow = ldg16(static_cast<const uint16_t*>(p.o) + oi);
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = bf_lo(ow[e]);
        o[2 * e + 1] = bf_hi(ow[e]);
      }
    }
    for (int e = 0; e < 4; ++e) acc += bf_lo(dw[e]) * o[2 * e] + bf_hi(dw[e]) * o[2 * e + 1];
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 8);
  if (sub == 0 && t < p.npad) {
    const int64_t bh = (int64_t)b * p.Hq + hq;
    const int64_t li = p.cu_seqlens ? (int64_t)hq * p.total_tokens + row : bh * p.N + t;
    p.delta[bh * p.npad + t] = t < sp.n ? acc : 0.f;
    p.lse2[bh * p.npad + t] = t < sp.n ? p.lse[li] * LOG2E : POS_INF;
  }
}

// An empty use of loaded registers: the loads must have completed here, so
// the tile loops that follow start with no register load in flight.
template <int N>
__device__ __forceinline__ void complete(const bf16x8 (&r)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : : "v"(r[i]));
}

// Plan entries (tile index, full-tile flag in bit 31) travel 64 at a time,
// one per lane, and are picked out with readlane.  A plain per-step load
// would have to complete before the tile loads that follow it in the same
// step can be left in flight.
struct PlanCursor {
  const int32_t* col;
  const uint8_t* flags;
  int end;
  int base;
  int chunk;
  __device__ int fetch(int b0, int lane) const {
    const int e = b0 + lane;
    return e < end ? (col[e] | (flags[e] ? (int)0x80000000 : 0)) : 0;
  }
  __device__ void init(const int32_t* c, const uint8_t* f, int e_begin, int e_end, int lane) {
    col = c;
    flags = f;
    end = e_end;
    base = e_begin;
    chunk = fetch(base, lane);
  }
  // entry e (wave-uniform); reloads the chunk when e leaves it
  __device__ int entry(int e, int lane) {
    if (e < base || e >= base + 64) {
      base = e;
      chunk = fetch(base, lane);
    }
    return __builtin_amdgcn_readlane(chunk, e - base);
  }
};

// ------------------------------------------------------------------- dQ --
constexpr int QBM = kFwdBlockM;  // 256 query rows per workgroup
constexpr int QBN = kFwdBlockN;  // 64 keys per tile
constexpr int QWAVES = QBM / 32;
constexpr int QTHREADS = 64 * QWAVES;

template <int D, bool GF32>
__global__ __attribute__((amdgpu_flat_work_group_size(QTHREADS, QTHREADS),
                          amdgpu_waves_per_eu(2, 2))) void cowa_bwd_dq_kernel(BwdParams p) {
  constexpr int CPR = D / 8, NK = D / 16, ND = D / 32;
  constexpr int TILE = QBN * D;
  constexpr int LOADS = QBN * CPR / 64 / QWAVES;
  static_assert(LOADS >= 1, "every wavefront loads part of each tile");
  // One LDS variable per buffer: the compiler tells distinct variables apart,
  // so the loads streaming into one buffer stay in flight while the step
  // reads the other (within one variable it would wait for them first).
  __shared__ __attribute__((aligned(16))) uint16_t K0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t K1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t V1[TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  const int per_b = p.nqt * p.Hq;
  const int wg = xcd_logical(blockIdx.x, p.xcd_chunk_q, p.B * per_b);
  if (wg < 0) return;
  const int b = wg / per_b;
  const int rem = wg - b * per_b;
  const int qi = p.nqt - 1 - rem / p.Hq;  // heavy first
  const int hq = rem - (rem / p.Hq) * p.Hq;
  const int h = hq / p.G;
  const HeadPattern hp = head_pattern(p.sink, p.window, p.band,
                                      band_slot(p.kv_head_offset + h, p.n_bands), p.causal);

  const SeqSpan sp = seq_span(p, b);
  if (qi * QBM >= sp.n) return;  // the whole workgroup: this tile is past the sequence
  const int q_row = qi * QBM + wave * 32 + l32;
  const int q_row_c = q_row < sp.n ? q_row : sp.n - 1;
  bf16x8 qf[NK], dof[NK];
  {
    const int64_t r = (int64_t)sp.start + q_row_c;
    const uint16_t* qp = p.q + (int64_t)b * p.qs_b + r * p.qs_t + (int64_t)hq * p.qs_h;
    const uint16_t* dp = p.dout + (int64_t)b * p.dos_b + r * p.dos_t + (int64_t)hq * p.dos_h;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, ldg16(qp + 16 * ks + 8 * hl));
      dof[ks] = __builtin_bit_cast(bf16x8, ldg16(dp + 16 * ks + 8 * hl));
    }
  }
  const int64_t bh = (int64_t)b * p.Hq + hq;
  const float lse2 = p.lse2[bh * p.npad + q_row_c];
  const float dlt = p.delta[bh * p.npad + q_row_c];

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};

  const int row = h * p.nqt + qi;
  const int e0 = p.row_ptr[row];
  const int e1 = p.row_ptr[row + 1];
  const uint16_t* kbase =
      p.k + (int64_t)b * p.ks_b + (int64_t)sp.start * p.ks_t + (int64_t)h * p.ks_h;
  const uint16_t* vbase =
      p.v + (int64_t)b * p.vs_b + (int64_t)sp.start * p.vs_t + (int64_t)h * p.vs_h;

  // lane offsets inside a tile are 32-bit (the host bounds 64 rows x stride
  // below 2^30 elements, so byte offsets stay below 2^31): the loads use a
  // buffer resource at the tile plus a 32-bit byte offset
  int ld_row[LOADS], ld_col[LOADS];
  uint32_t ld_koff[LOADS], ld_voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int P = (wave * LOADS + i) * 64 + lane;
    ld_row[i] = P / CPR;
    ld_col[i] = ((P % CPR) ^ swz_both<D>(ld_row[i])) * 8;
    ld_koff[i] = (uint32_t)(ld_row[i] * p.ks_t) + ld_col[i];
    ld_voff[i] = (uint32_t)(ld_row[i] * p.vs_t) + ld_col[i];
  }
  // K and V tiles of key tile kj into buffer slot; keys past N (only in
  // tiles the plan marks partial, where they are masked) are clamped.
  auto load_kv = [&](int kj, uint16_t* kd, uint16_t* vd) {
    const int key0 = kj * QBN;
    const __amdgpu_buffer_rsrc_t kr = lds_rsrc(kbase + (int64_t)key0 * p.ks_t);
    const __amdgpu_buffer_rsrc_t vr = lds_rsrc(vbase + (int64_t)key0 * p.vs_t);
    if (key0 + QBN <= sp.n) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        buf2lds16(kr, (int)(ld_koff[i] * 2), kd + (wave * LOADS + i) * 512);
        buf2lds16(vr, (int)(ld_voff[i] * 2), vd + (wave * LOADS + i) * 512);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        int key = key0 + ld_row[i];
        key = key < sp.n ? key : sp.n - 1;
        buf2lds16(kr, (int)(((key - key0) * p.ks_t + ld_col[i]) * 2),
                  kd + (wave * LOADS + i) * 512);
        buf2lds16(vr, (int)(((key - key0) * p.vs_t + ld_col[i]) * 2),
                  vd + (wave * LOADS + i) * 512);
      }
    }
  };

  int n_off[2][NK], t_off[2][ND];
  plain_offsets<D>(l32, hl, n_off);
  tr_offsets<D>(lane, t_off);

  PlanCursor pc;
  pc.init(p.col, p.flags, e0, e1, lane);
  // The register operands and the first plan chunk are complete on every path
  // into the tile loop (otherwise the loop waits for its own prefetch).
  complete(qf);
  complete(dof);
  asm volatile("" : : "v"(lse2), "v"(dlt), "v"(pc.chunk));

  int c_cur = 0;
  if (e0 < e1) {
    c_cur = pc.entry(e0, lane);
    load_kv(c_cur & 0x7fffffff, K0, V0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // One step on the tiles in (Ks, Vs) while the next ones stream into (Kn, Vn).
  auto step = [&](int e, const uint16_t* Ks, const uint16_t* Vs, uint16_t* Kn, uint16_t* Vn) {
    int c_nxt = 0;
    if (e + 1 < e1) {
      c_nxt = pc.entry(e + 1, lane);
      load_kv(c_nxt & 0x7fffffff, Kn, Vn);
    }
    const int kj = c_cur & 0x7fffffff;
    const bool full = c_cur < 0;

#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      unsigned pk[8];
      f32x16 s = f32x16{}, dpv = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + n_off[blk][ks]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vs + n_off[blk][ks]);
        dpv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dof[ks], dpv, 0, 0, 0);
      }
      if (!full) {
        // register i holds key kj*64 + 4 hl + 32 blk + 8 (i/4) + i%4
        const uint64_t vis = row_visible_bits(hp, q_row, kj * QBN + 4 * hl);
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = keep_if(s[i], vis, 32 * blk + 8 * (i >> 2) + (i & 3));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i], p.scale_log2, -lse2));
        const float p1 =
            __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i + 1], p.scale_log2, -lse2));
        pk[i] = pack_bf16(p0 * (dpv[2 * i] - dlt), p1 * (dpv[2 * i + 1] - dlt));
      }
      // dQ^T += K^T dS^T over this block's 32 keys (two 16-key steps)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int st = 2 * blk + half, o4 = half * 4;
        const u32x4 w = {pk[o4], pk[o4 + 1], pk[o4 + 2], pk[o4 + 3]};
        const bf16x8 bv = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const bf16x8 a =
              lds_read_tr_pair(Ks + st * 16 * D + t_off[0][db], Ks + st * 16 * D + t_off[1][db]);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[db], 0, 0, 0);
        }
      }
    }
    c_cur = c_nxt;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int e = e0; e < e1; e += 2) {
    step(e, K0, V0, K1, V1);
    if (e + 1 < e1) step(e + 1, K1, V1, K0, V0);
  }

  if (q_row < sp.n) {
    char* gbase = reinterpret_cast<char*>(p.dq);
    const int64_t gi = (int64_t)b * p.dqs_b + ((int64_t)sp.start + q_row) * p.dqs_t +
                       (int64_t)hq * p.dqs_h;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dd = 32 * db + 8 * g4 + 4 * hl;
        const float v0 = acc[db][4 * g4] * p.scale, v1 = acc[db][4 * g4 + 1] * p.scale;
        const float v2 = acc[db][4 * g4 + 2] * p.scale, v3 = acc[db][4 * g4 + 3] * p.scale;
        if (GF32)
          *reinterpret_cast<f32x4*>(gbase + (gi + dd) * 4) = f32x4{v0, v1, v2, v3};
        else
          *reinterpret_cast<u32x2*>(gbase + (gi + dd) * 2) =
              u32x2{pack_bf16(v0, v1), pack_bf16(v2, v3)};
      }
  }
}

// ---------------------------------------------------------------- dK/dV --
constexpr int KBM = kBwdBlockM;  // 64 query rows per step
constexpr int KBN = kBwdBlockN;  // 128 keys per workgroup
constexpr int KWAVES = KBN / 32;
constexpr int KTHREADS = 64 * KWAVES;

template <int D, bool GF32>
__device__ __forceinline__ void store_key_row(void* base, int64_t idx, const f32x16* acc,
                                              float mul, int hl) {
  constexpr int ND = D / 32;
  char* g = reinterpret_cast<char*>(base);
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int dd = 32 * db + 8 * g4 + 4 * hl;
      const float v0 = acc[db][4 * g4] * mul, v1 = acc[db][4 * g4 + 1] * mul;
      const float v2 = acc[db][4 * g4 + 2] * mul, v3 = acc[db][4 * g4 + 3] * mul;
      if (GF32)
        *reinterpret_cast<f32x4*>(g + (idx + dd) * 4) = f32x4{v0, v1, v2, v3};
      else
        *reinterpret_cast<u32x2*>(g + (idx + dd) * 2) =
            u32x2{pack_bf16(v0, v1), pack_bf16(v2, v3)};
    }
}

template <int D, bool GF32>
__global__ __attribute__((amdgpu_flat_work_group_size(KTHREADS, KTHREADS),
                          amdgpu_waves_per_eu(1, 1))) void cowa_bwd_dkdv_kernel(BwdParams p) {
  constexpr int CPR = D / 8, NK = D / 16, ND = D / 32;
  constexpr int TILE = KBM * D;
  constexpr int LOADS = KBM * CPR / 64 / KWAVES;
  static_assert(LOADS >= 1, "every wavefront loads part of each tile");
  // one LDS variable per buffer (as in the dQ kernel); S0, S1 hold LSE2 then D
  __shared__ __attribute__((aligned(16))) uint16_t Q0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t Q1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t O0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t O1[TILE];
  __shared__ __attribute__((aligned(16))) float S0[2 * KBM];
  __shared__ __attribute__((aligned(16))) float S1[2 * KBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  // First the parts of the split sink key tiles, then the other key tiles in
  // ascending order (in causal mode the early ones carry the most query tiles).
  const int n_part_wg = p.B * p.Hkv * p.n_sink_tiles * p.nch;
  int wg = xcd_logical(blockIdx.x, p.xcd_chunk_kv,
                       p.B * p.Hkv * (p.nkt_kv + p.n_sink_tiles * (p.nch - 1)));
  if (wg < 0) return;
  int b, h, kj, part = -1;
  if (wg < n_part_wg) {
    part = wg % p.nch;
    int t = wg / p.nch;
    kj = t % p.n_sink_tiles;
    t /= p.n_sink_tiles;
    h = t % p.Hkv;
    b = t / p.Hkv;
  } else {
    wg -= n_part_wg;
    const int per_kj = p.B * p.Hkv;
    kj = p.n_sink_tiles + wg / per_kj;
    const int rem = wg % per_kj;
    b = rem / p.Hkv;
    h = rem - b * p.Hkv;
  }
  const HeadPattern hp = head_pattern(p.sink, p.window, p.band,
                                      band_slot(p.kv_head_offset + h, p.n_bands), p.causal);

  const SeqSpan sp = seq_span(p, b);
  if (kj * KBN >= sp.n) return;  // the whole workgroup: this tile is past the sequence
  const int key = kj * KBN + wave * 32 + l32;
  const int key_c = key < sp.n ? key : sp.n - 1;
  bf16x8 kf[NK], vf[NK];
  {
    const int64_t r = (int64_t)sp.start + key_c;
    const uint16_t* kp = p.k + (int64_t)b * p.ks_b + r * p.ks_t + (int64_t)h * p.ks_h;
    const uint16_t* vp = p.v + (int64_t)b * p.vs_b + r * p.vs_t + (int64_t)h * p.vs_h;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      kf[ks] = __builtin_bit_cast(bf16x8, ldg16(kp + 16 * ks + 8 * hl));
      vf[ks] = __builtin_bit_cast(bf16x8, ldg16(vp + 16 * ks + 8 * hl));
    }
  }
  // The accumulators start as the (zero) result of an MFMA rather than as
  // zero constants: the compiler then keeps them in accumulator registers
  // across the step loop, where the MFMAs update them in place (started from
  // constants, every step copied all 128 values out to ordinary registers
  // and back).
  f32x16 dk[ND], dv[ND];
  {
    const bf16x8 z = {};
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      dk[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z, z, f32x16{}, 0, 0, 0);
      dv[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z, z, f32x16{}, 0, 0, 0);
    }
  }

  // steps run over (query head of the group, visible query tile); a part
  // takes one contiguous range of them
  const int r = h * p.nkt_kv + kj;
  const int e0 = p.row_ptr_kv[r];
  int e1 = p.row_ptr_kv[r + 1];
  if (p.cu_seqlens) {
    // the plan is built for the longest sequence: keep the query tiles that
    // start inside this one (the list is ascending)
    const int nq = (sp.n + KBM - 1) / KBM;
    int lo = e0, hi = e1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (p.col_kv[mid] < nq) lo = mid + 1;
      else hi = mid;
    }
    e1 = lo;
  }
  const int cnt = e1 - e0;
  const int total = cnt * p.G;
  int s_begin = 0, s_end = total;
  if (part >= 0) {
    const int len = (total + p.nch - 1) / p.nch;
    s_begin = min(total, part * len);
    s_end = min(total, s_begin + len);
  }
  const int nsteps = s_end - s_begin;

  int ld_row[LOADS], ld_col[LOADS];
  uint32_t ld_qoff[LOADS], ld_ooff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int P = (wave * LOADS + i) * 64 + lane;
    ld_row[i] = P / CPR;
    ld_col[i] = ((P % CPR) ^ swz_both<D>(ld_row[i])) * 8;
    ld_qoff[i] = (uint32_t)(ld_row[i] * p.qs_t) + ld_col[i];
    ld_ooff[i] = (uint32_t)(ld_row[i] * p.dos_t) + ld_col[i];
  }
  // Q and dO rows of query tile qi of head hq into buffer slot, with that
  // tile's LSE2 and D; rows past N are clamped (their LSE2 is +inf).
  auto load_q = [&](int hq, int qi, uint16_t* qd, uint16_t* od, float* sdst) {
    const int r0 = qi * KBM;
    const uint16_t* qb =
        p.q + (int64_t)b * p.qs_b + (int64_t)sp.start * p.qs_t + (int64_t)hq * p.qs_h;
    const uint16_t* ob =
        p.dout + (int64_t)b * p.dos_b + (int64_t)sp.start * p.dos_t + (int64_t)hq * p.dos_h;
    const __amdgpu_buffer_rsrc_t qr = lds_rsrc(qb + (int64_t)r0 * p.qs_t);
    const __amdgpu_buffer_rsrc_t orr = lds_rsrc(ob + (int64_t)r0 * p.dos_t);
    if (r0 + KBM <= sp.n) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        buf2lds16(qr, (int)(ld_qoff[i] * 2), qd + (wave * LOADS + i) * 512);
        buf2lds16(orr, (int)(ld_ooff[i] * 2), od + (wave * LOADS + i) * 512);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        int t = r0 + ld_row[i];
        t = t < sp.n ? t : sp.n - 1;
        buf2lds16(qr, (int)(((t - r0) * p.qs_t + ld_col[i]) * 2), qd + (wave * LOADS + i) * 512);
        buf2lds16(orr, (int)(((t - r0) * p.dos_t + ld_col[i]) * 2),
                  od + (wave * LOADS + i) * 512);
      }
    }
    const int64_t so = ((int64_t)b * p.Hq + hq) * p.npad + r0;
    if (wave == 0) buf2lds4(lds_rsrc(p.lse2 + so), lane * 4, sdst);
    if (wave == 1) buf2lds4(lds_rsrc(p.delta + so), lane * 4, sdst + KBM);
  };

  int n_off[2][NK], t_off[2][ND];
  plain_offsets<D>(l32, hl, n_off);
  tr_offsets<D>(lane, t_off);

  int hq_cur = h * p.G, e_cur = e0, c_cur = 0;
  if (cnt > 0) {
    hq_cur += s_begin / cnt;
    e_cur += s_begin % cnt;
  }
  PlanCursor pc;
  pc.init(p.col_kv, p.flags_kv, e_cur, e1, lane);
  // K, V registers and the first plan chunk complete on every path into the loop
  complete(kf);
  complete(vf);
  asm volatile("" : : "v"(pc.chunk));
  if (nsteps > 0) {
    c_cur = pc.entry(e_cur, lane);
    load_q(hq_cur, c_cur & 0x7fffffff, Q0, O0, S0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // One step on the tiles in (Qs, Os, Ss) while the next ones stream into
  // (Qn, On, Sn).
  auto step = [&](int s, const uint16_t* Qs, const uint16_t* Os, const float* Ss, uint16_t* Qn,
                  uint16_t* On, float* Sn) {
    const float* sl = Ss;
    const float* sd = Ss + KBM;
    int hq_nxt = hq_cur, e_nxt = e_cur + 1, c_nxt = 0;
    if (e_nxt == e1) {
      e_nxt = e0;
      ++hq_nxt;
    }
    if (s + 1 < nsteps) {
      c_nxt = pc.entry(e_nxt, lane);
      load_q(hq_nxt, c_nxt & 0x7fffffff, Qn, On, Sn);
    }
    const int qi = c_cur & 0x7fffffff;
    const bool full = c_cur < 0;

#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      unsigned pp[8], ps[8];
      f32x16 sv = f32x16{}, dpv = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Qs + n_off[blk][ks]);
        sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ks], sv, 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Os + n_off[blk][ks]);
        dpv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[ks], dpv, 0, 0, 0);
      }
      if (!full) {
        // register i holds query qi*64 + 4 hl + 32 blk + 8 (i/4) + i%4
        const uint64_t vis = col_visible_bits(hp, qi * KBM + 4 * hl, key);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sv[i] = keep_if(sv[i], vis, 32 * blk + 8 * (i >> 2) + (i & 3));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + 32 * blk + 8 * j + 4 * hl);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sd + 32 * blk + 8 * j + 4 * hl);
        float pv[4], dsv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          pv[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[4 * j + u], p.scale_log2, -l4[u]));
          dsv[u] = pv[u] * (dpv[4 * j + u] - d4[u]);
        }
        pp[2 * j] = pack_bf16(pv[0], pv[1]);
        pp[2 * j + 1] = pack_bf16(pv[2], pv[3]);
        ps[2 * j] = pack_bf16(dsv[0], dsv[1]);
        ps[2 * j + 1] = pack_bf16(dsv[2], dsv[3]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over this block's 32 query rows
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int st = 2 * blk + half, o4 = half * 4;
        const u32x4 wp = {pp[o4], pp[o4 + 1], pp[o4 + 2], pp[o4 + 3]};
        const u32x4 ws = {ps[o4], ps[o4 + 1], ps[o4 + 2], ps[o4 + 3]};
        const bf16x8 bp = __builtin_bit_cast(bf16x8, wp);
        const bf16x8 bs = __builtin_bit_cast(bf16x8, ws);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const bf16x8 a = lds_read_tr_pair(Os + st * 16 * D + t_off[0][db],
                                            Os + st * 16 * D + t_off[1][db]);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp, dv[db], 0, 0, 0);
        }
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          const bf16x8 a = lds_read_tr_pair(Qs + st * 16 * D + t_off[0][db],
                                            Qs + st * 16 * D + t_off[1][db]);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bs, dk[db], 0, 0, 0);
        }
      }
    }
    hq_cur = hq_nxt;
    e_cur = e_nxt;
    c_cur = c_nxt;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // unrolled by two so the buffers alternate with compile-time slots
  for (int s = 0; s < nsteps; s += 2) {
    step(s, Q0, O0, S0, Q1, O1, S1);
    if (s + 1 < nsteps) step(s + 1, Q1, O1, S1, Q0, O0, S0);
  }

  if (part >= 0) {
    // fp32 partials [b][h][sink tile][part][dK, dV][key][d]
    const int64_t slot =
        (((int64_t)(b * p.Hkv + h) * p.n_sink_tiles + kj) * p.nch + part) * 2;
    const int64_t row = (int64_t)(wave * 32 + l32) * D;
    store_key_row<D, true>(p.part, slot * KBN * D + row, dk, p.scale, hl);
    store_key_row<D, true>(p.part, (slot + 1) * KBN * D + row, dv, 1.f, hl);
  } else if (key < sp.n) {
    const int64_t row = (int64_t)sp.start + key;
    store_key_row<D, GF32>(p.dk, (int64_t)b * p.dks_b + row * p.dks_t + (int64_t)h * p.dks_h,
                           dk, p.scale, hl);
    store_key_row<D, GF32>(p.dv, (int64_t)b * p.dvs_b + row * p.dvs_t + (int64_t)h * p.dvs_h,
                           dv, 1.f, hl);
  }
}

// Sum of the parts of the split sink key tiles, in part order.  Grid
// (H_kv * n_sink_tiles * reduce_split(D), B); each thread covers 8 head dims
// of one key, each workgroup 256 / (D / 8) keys.
constexpr int reduce_split(int d) { return KBN * (d / 8) / 256; }
template <int D, bool GF32>
__global__ __launch_bounds__(256) void cowa_bwd_part_reduce_kernel(BwdParams p) {
  constexpr int REDUCE_SPLIT = reduce_split(D);
  const int t = blockIdx.x / REDUCE_SPLIT;
  const int kj = t % p.n_sink_tiles;
  const int h = t / p.n_sink_tiles;
  const int b = blockIdx.y;
  const int64_t slot0 = (((int64_t)(b * p.Hkv + h) * p.n_sink_tiles + kj) * p.nch) * 2;
  {
    const int u = (blockIdx.x % REDUCE_SPLIT) * 256 + threadIdx.x;  // key x (D / 8) chunks
    const int kl = u / (D / 8);
    const int d0 = (u % (D / 8)) * 8;
    const int key = kj * KBN + kl;
    const SeqSpan sp = seq_span(p, b);
    if (key >= sp.n) return;
    const int64_t row = (int64_t)sp.start + key;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      f32x4 a = {}, c = {};
      for (int part = 0; part < p.nch; ++part) {
        const float* src = p.part + ((slot0 + 2 * part + which) * KBN + kl) * D + d0;
        a += *reinterpret_cast<const f32x4*>(src);
        c += *reinterpret_cast<const f32x4*>(src + 4);
      }
      void* dst = which == 0 ? p.dk : p.dv;
      const int64_t idx = which == 0
          ? (int64_t)b * p.dks_b + row * p.dks_t + (int64_t)h * p.dks_h + d0
          : (int64_t)b * p.dvs_b + row * p.dvs_t + (int64_t)h * p.dvs_h + d0;
      if (GF32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + idx) = a;
        *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + idx + 4) = c;
      } else {
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + idx) =
            u32x4{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(c[0], c[1]),
                  pack_bf16(c[2], c[3])};
      }
    }
  }
}

template <int D>
int launch_bwd_d(const BwdParams& p_in, hipStream_t s) {
  // XCD chunks: up to 8 query tiles with all their heads (dQ); up to
  // KV_CHUNK_TILES key tiles with all their (sequence, head) pairs (dK/dV)
  BwdParams p = p_in;
  const int64_t kv_units = p.nkt_kv + (int64_t)p.n_sink_tiles * (p.nch - 1);
  if (p.xcd_chunk_q <= 0) p.xcd_chunk_q = xcd_chunk(p.Hq, (int64_t)p.B * p.nqt, 8);
  if (p.xcd_chunk_kv <= 0)
    p.xcd_chunk_kv = xcd_chunk((int64_t)p.B * p.Hkv, kv_units, KV_CHUNK_TILES);
  hipLaunchKernelGGL(cowa_bwd_delta_kernel<D>, dim3((unsigned)(p.npad / DELTA_ROWS), p.Hq, p.B),
                     dim3(256), 0, s, p);
  const dim3 gq((unsigned)xcd_grid((int64_t)p.B * p.nqt * p.Hq, p.xcd_chunk_q));
  const dim3 gk((unsigned)xcd_grid((int64_t)p.B * p.Hkv * kv_units, p.xcd_chunk_kv));
  const dim3 gr((unsigned)(p.Hkv * p.n_sink_tiles * reduce_split(D)), (unsigned)p.B);
  if (p.g_f32) {
    hipLaunchKernelGGL((cowa_bwd_dq_kernel<D, true>), gq, dim3(QTHREADS), 0, s, p);
    hipLaunchKernelGGL((cowa_bwd_dkdv_kernel<D, true>), gk, dim3(KTHREADS), 0, s, p);
    if (p.n_sink_tiles > 0)
      hipLaunchKernelGGL((cowa_bwd_part_reduce_kernel<D, true>), gr, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((cowa_bwd_dq_kernel<D, false>), gq, dim3(QTHREADS), 0, s, p);
    hipLaunchKernelGGL((cowa_bwd_dkdv_kernel<D, false>), gk, dim3(KTHREADS), 0, s, p);
    if (p.n_sink_tiles > 0)
      hipLaunchKernelGGL((cowa_bwd_part_reduce_kernel<D, false>), gr, dim3(256), 0, s, p);
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_bwd(const BwdParams& p, int d, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d == 128) return launch_bwd_d<128>(p, s);
  if (d == 64) return launch_bwd_d<64>(p, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace cowa
