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
// Workgroup = 4 wavefronts = 128 query rows of one (batch, query head).
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
// swizzled by the row index so that 16 consecutive rows read at one column
// hit distinct banks.  K feeds the first product with 16-byte reads; V feeds
// the second through the gfx950 transposing read (ds_read_b64_tr_b16), which
// hands each lane four keys of one head dimension.
#include <hip/hip_runtime.h>

#include "cowa_internal.h"

namespace cowa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kFwdBlockM;  // 128 query rows per workgroup
constexpr int BN = kFwdBlockN;  // 64 keys per tile
constexpr int NTHREADS = 256;
constexpr float NEG_INF = -__builtin_huge_valf();

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Lane l and lane l^32 hold the two halves of one query column; this returns
// (value of lane l, value of lane l^32) in some order on every lane.
__device__ __forceinline__ void pair_swap(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_swap(x, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_swap(x, a, b);
  return a + b;
}

// The running maximum is only raised when a row's maximum grows by more than
// 2^RESCALE_LOG2 in probability terms; until then the stale maximum is kept
// and probabilities may reach 2^RESCALE_LOG2 (exact: the same reference
// maximum is used for the sum and for the output).
constexpr float RESCALE_LOG2 = 8.0f;

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  bf16x2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, r);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One 16-byte chunk per lane from global memory straight into LDS; the
// wavefront's 64 chunks land contiguously at lds_base (+16 bytes per lane).
__device__ __forceinline__ void g2lds16(const uint16_t* g, uint16_t* lds_base) {
  __builtin_amdgcn_global_load_lds((const void*)g, (lds_void*)lds_base, 16, 0, 0);
}

__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

template <int D, bool OF32>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2, 2))) void cowa_fwd_kernel(FwdParams p) {
  constexpr int CPR = D / 8;                  // 16-byte chunks per K/V row
  constexpr int TILE = BN * D;                // bf16 elements per K or V tile
  constexpr int LOADS = BN * CPR / 64 / 4;    // direct loads per wave per tile
  constexpr int ND = D / 32;                  // 32-wide d blocks of O^T
  constexpr int NK = D / 16;                  // 16-deep k steps of Q.K

  // [buffer][K tile, V tile]
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  // heavy-first order: later query tiles see more keys
  const int per_b = p.nqt * p.Hq;
  const int wg = blockIdx.x;
  const int b = wg / per_b;
  const int rem = wg - b * per_b;
  const int qi = p.nqt - 1 - rem / p.Hq;
  const int hq = rem - (rem / p.Hq) * p.Hq;
  const int h = hq / p.G;
  const HeadPattern hp = head_pattern(p.sink, p.window, p.band, p.kv_head_offset + h, p.causal);

  const int q_row = qi * BM + wave * 32 + l32;
  const int q_row_c = q_row < p.N ? q_row : p.N - 1;

  bf16x8 qf[NK];
  {
    const uint16_t* qp = p.q + (int64_t)b * p.qs_b + (int64_t)q_row_c * p.qs_t + (int64_t)hq * p.qs_h;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, ldg16(qp + 16 * ks + 8 * hl));
  }

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};
  float m_run = NEG_INF;
  float l_run = 0.f;

  const int row = h * p.nqt + qi;
  const int e0 = p.row_ptr[row];
  const int e1 = p.row_ptr[row + 1];
  const uint16_t* kbase = p.k + (int64_t)b * p.ks_b + (int64_t)h * p.ks_h;
  const uint16_t* vbase = p.v + (int64_t)b * p.vs_b + (int64_t)h * p.vs_h;

  // Direct-load geometry: LDS chunk position P = (wave*LOADS + i)*64 + lane
  // holds row P / CPR, column chunk (P % CPR) ^ (row % CPR).
  int ld_row[LOADS], ld_col[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int P = (wave * LOADS + i) * 64 + lane;
    ld_row[i] = P / CPR;
    ld_col[i] = ((P % CPR) ^ (ld_row[i] % CPR)) * 8;
  }
  // Keys past N are clamped to N - 1: such keys only occur in tiles the plan
  // marks partial, where they are masked (their probability is exactly 0).
  auto issue_loads = [&](int kj, int buf) {
    const int key0 = kj * BN;
    uint16_t* Ks = smem + buf * 2 * TILE;
    uint16_t* Vs = Ks + TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      int key = key0 + ld_row[i];
      key = key < p.N ? key : p.N - 1;
      const int off = (wave * LOADS + i) * 64 * 8;
      g2lds16(kbase + (int64_t)key * p.ks_t + ld_col[i], Ks + off);
      g2lds16(vbase + (int64_t)key * p.vs_t + ld_col[i], Vs + off);
    }
  };

  // K read offsets (first product, A operand): row 32*blk + l32, chunk 2*ks + hl
  int k_off[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) k_off[ks] = l32 * D + (((2 * ks + hl) ^ (l32 % CPR)) * 8);
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
      v_off[ri][db] = key * D + (((d >> 3) ^ (key % CPR)) * 8) + (d & 7);
    }

  if (e0 < e1) issue_loads(p.col[e0], 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int e = e0; e < e1; ++e) {
    const int buf = (e - e0) & 1;
    const int kj = p.col[e];
    const bool full = p.flags[e] != 0;
    if (e + 1 < e1) issue_loads(p.col[e + 1], buf ^ 1);

    const uint16_t* Ks = smem + buf * 2 * TILE;
    const uint16_t* Vs = Ks + TILE;

    // S^T for keys [32*blk, 32*blk+32) of the tile
    f32x16 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + blk * 32 * D + k_off[ks]);
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[blk], 0, 0, 0);
      }
    }

    if (!full) {
      const int key0 = kj * BN + 4 * hl;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * blk + 8 * (i >> 2) + (i & 3);
          if (!visible(hp, q_row, key)) s[blk][i] = NEG_INF;
        }
    }

    float mt = NEG_INF;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[blk][i]);
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
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[blk][i], p.scale_log2, -mb));
        s[blk][i] = e2;
        l_run += e2;
      }

    // O^T += V^T P^T, four 16-key steps
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int blk = st >> 1;
      const int o8 = (st & 1) * 8;
      u32x4 pw;
      pw.x = pack_bf16(s[blk][o8 + 0], s[blk][o8 + 1]);
      pw.y = pack_bf16(s[blk][o8 + 2], s[blk][o8 + 3]);
      pw.z = pack_bf16(s[blk][o8 + 4], s[blk][o8 + 5]);
      pw.w = pack_bf16(s[blk][o8 + 6], s[blk][o8 + 7]);
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

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  const float l_tot = pair_sum(l_run);
  if (q_row < p.N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    char* obase = reinterpret_cast<char*>(p.o);
    const int64_t oidx = (int64_t)b * p.os_b + (int64_t)q_row * p.os_t + (int64_t)hq * p.os_h;
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
      p.lse[((int64_t)b * p.Hq + hq) * p.N + q_row] = lse;
    }
  }
}

}  // namespace

int launch_fwd(const FwdParams& p, int d, int o_f32, void* stream) {
  const dim3 grid((unsigned)((int64_t)p.B * p.nqt * p.Hq));
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
