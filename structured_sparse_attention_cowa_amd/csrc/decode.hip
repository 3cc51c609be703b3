// CoWA single-token decode for gfx950: split-KV, HBM-streaming, two kernels.
//
// The decode query of sequence b sits at t = len_b - 1 and sees, per KV head
// g, the same visible set as prefill row t: shared sink, shared local window
// and band g ("CoWindow Attention: Full Causal Coverage Is a Collective
// Property", Abstract: one pattern for training and inference).  Those keys
// form at most three disjoint ranges; the split kernel walks their
// concatenation in chunks, so only visible K/V rows are ever read.
//
// Split kernel, one workgroup per (chunk, KV head, sequence), 4 wavefronts:
//   phase A  8 lanes per key (d/8 dims each) dot the key with all G query
//            heads of the KV head (packed bf16 dot products, 8-lane DPP
//            reduction) and store scaled scores in LDS;
//   phase B  block max per head, then p = exp2(s - max) in LDS and the row
//            sums;
//   phase C  d/8 lanes per key (8 dims each) accumulate p * v for the G heads
//            in fp32, reduced across lanes and wavefronts at the end.
// The chunk's normalised output and log-sum-exp go to the workspace.
// Combine kernel, one workgroup per (sequence, query head): merges the chunks
// by their log-sum-exp, weights staged in LDS, partial loads all in flight.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cowa_internal.h"

namespace cowa {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NTHREADS = 256;
constexpr int NWAVES = 4;
constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float LN2 = 0.69314718055994531f;

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Cross-lane steps on the DPP path (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xb1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4e;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7 - i within 8 lanes

// Sum over aligned groups of 8 lanes, result on every lane of the group.
__device__ __forceinline__ float sum8(float a) {
  a += dpp<DPP_XOR1>(a);
  a += dpp<DPP_XOR2>(a);
  return a + dpp<DPP_HALF_MIRROR>(a);
}


struct Segs {
  int lo0, n0, lo1, n1, lo2, n2;
  // windowed layout (ring > 0): ring rows follow s_rows sink rows; rs1, rs2
  // are the ring rows of the band and local ranges' first keys
  int ring, s_rows, rs1, rs2;
  // cache row of the v-th visible key (its position in the full layout);
  // each non-sink range is at most one ring long, so it wraps at most once
  __device__ int row(int v) const {
    if (ring == 0) return key(v);
    if (v < n0) return lo0 + v;
    v -= n0;
    int r = v < n1 ? rs1 + v : rs2 + (v - n1);
    r = r >= ring ? r - ring : r;
    return s_rows + r;
  }
  __device__ int key(int v) const {
    if (v < n0) return lo0 + v;
    v -= n0;
    if (v < n1) return lo1 + v;
    return lo2 + v - n1;
  }
  __device__ int total() const { return n0 + n1 + n2; }
};

__device__ __forceinline__ Segs decode_segs(const DecodeParams& p, int b, int h, int* t_out) {
  int len = p.seqlens[b];
  len = len < 1 ? 1 : (len > p.n_max ? p.n_max : len);
  const int t = len - 1;
  const HeadPattern hp = head_pattern(p.sink, p.window, p.band,
                                      band_slot(p.kv_head_offset + h, p.n_bands), p.causal);
  const RowRanges rr = row_ranges(hp, t);
  Segs s;
  s.lo0 = rr.lo[0];
  s.n0 = rr.hi[0] - rr.lo[0];
  s.lo1 = rr.lo[1];
  s.n1 = rr.hi[1] - rr.lo[1];
  s.lo2 = rr.lo[2];
  s.n2 = rr.hi[2] - rr.lo[2];
  s.ring = 0;
  s.s_rows = 0;
  s.rs1 = s.rs2 = 0;
  if (p.win) {
    s.s_rows = window_sink_rows(p.sink, p.n_max);
    s.ring = window_ring_rows(p.sink, p.window, p.band,
                              band_slot(p.kv_head_offset + h, p.n_bands), p.n_max);
    if (s.ring > 0) {
      s.rs1 = s.n1 > 0 ? (s.lo1 - s.s_rows) % s.ring : 0;
      s.rs2 = s.n2 > 0 ? (s.lo2 - s.s_rows) % s.ring : 0;
    }
  }
  *t_out = t;
  return s;
}

// First row of local KV head h in a windowed cache (heads are stacked).
__device__ __forceinline__ int64_t window_head_row(const DecodeParams& p, int h) {
  const int s_rows = window_sink_rows(p.sink, p.n_max);
  int64_t r = 0;
  for (int i = 0; i < h; ++i)
    r += s_rows + window_ring_rows(p.sink, p.window, p.band,
                                   band_slot(p.kv_head_offset + i, p.n_bands), p.n_max);
  return r;
}

// Cache rows are read once per step: non-temporal loads (the `nt` cache
// policy) stream them without keeping them in L2, 3-4% faster than ordinary
// loads at the 128K, 16-sequence decode step.
__device__ __forceinline__ u32x4 ldg16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int D, int G>
__global__ __launch_bounds__(NTHREADS) void cowa_decode_split(DecodeParams p) {
  constexpr int GP = (G + 3) / 4 * 4;   // padded head count of an LDS score row
  constexpr int LPA = 8;                // phase A: lanes per key
  constexpr int KPA = 64 / LPA;         // phase A: keys per wavefront step
  constexpr int DPL = D / LPA;          // phase A: dims per lane
  constexpr int NVA = DPL / 8;          // phase A: 16-byte loads per lane
  constexpr int LPV = D / 8;            // phase C: lanes per key
  constexpr int KPW = 64 / LPV;         // phase C: keys per wavefront step
  constexpr int UA = 4;                 // phase A unroll (keys per lane group in flight)
  constexpr int UC = 6;                 // phase C unroll

  __shared__ __attribute__((aligned(16))) float sc[kDecodeChunkMax * GP];
  __shared__ float red[NWAVES][GP];
  __shared__ float stat_m[GP];
  __shared__ float stat_l[GP];
  __shared__ __attribute__((aligned(16))) float accs[NWAVES][G * D];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  int t;
  const Segs sg = decode_segs(p, b, h, &t);
  const int nvis = sg.total();
  const int v0 = split * p.chunk;
  if (v0 >= nvis) return;
  const int cnt = (nvis - v0) < p.chunk ? (nvis - v0) : p.chunk;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int64_t hrow = p.win ? window_head_row(p, h) : 0;
  const uint16_t* kbase = p.k + (int64_t)b * p.ks_b + (p.win ? hrow * p.ks_t : (int64_t)h * p.ks_h);
  const uint16_t* vbase = p.v + (int64_t)b * p.vs_b + (p.win ? hrow * p.vs_t : (int64_t)h * p.vs_h);

  // ---- phase A: scores ----
  {
    const int quad = lane / LPA;   // key slot of this lane
    // dims 8 part + 8 LPA i + (0..7), i < NVA: each 16-byte load of the
    // eight lanes of a key covers one whole 128-byte line of its row (two
    // loads of adjacent 16-byte pieces per lane read 10% slower)
    const int part = lane % LPA;
    u32x4 qr[G][NVA];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint16_t* qp = p.q + (int64_t)b * p.qs_b + (int64_t)(h * G + hh) * p.qs_h + part * 8;
#pragma unroll
      for (int i = 0; i < NVA; ++i) qr[hh][i] = ldg16(qp + 8 * LPA * i);
    }
    float mx[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) mx[hh] = NEG_INF;

    for (int base = wave * KPA + quad; base < cnt; base += NWAVES * KPA * UA) {
      u32x4 kr[UA][NVA];
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int kk = base + NWAVES * KPA * u;
        if (kk < cnt) {
          const int key = sg.row(v0 + kk);
          const uint16_t* kp = kbase + (int64_t)key * p.ks_t + part * 8;
#pragma unroll
          for (int i = 0; i < NVA; ++i) kr[u][i] = ldg16_stream(kp + 8 * LPA * i);
        }
      }
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int kk = base + NWAVES * KPA * u;
        if (kk < cnt) {
          float sv[G];
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < NVA; ++i)
#pragma unroll
              for (int w = 0; w < 4; ++w) a = dot2(kr[u][i][w], qr[hh][i][w], a);
            a = sum8(a);
            sv[hh] = a * p.scale_log2;
            mx[hh] = fmaxf(mx[hh], sv[hh]);
          }
#pragma unroll
          for (int hh = 0; hh < G; ++hh)
            if ((hh % LPA) == part) sc[kk * GP + hh] = sv[hh];
        }
      }
    }
    // wave max over the 16 quads, then across waves
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float m = mx[hh];
#pragma unroll
      for (int off = LPA; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
      if (lane == 0) red[wave][hh] = m;
    }
  }
  __syncthreads();
  if (tid < G) {
    float m = red[0][tid];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) m = fmaxf(m, red[w][tid]);
    stat_m[tid] = m;
  }
  __syncthreads();

  // ---- phase B: probabilities and row sums ----
  {
    float ls[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) ls[hh] = 0.f;
    for (int kk = tid; kk < cnt; kk += NTHREADS) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float e = __builtin_amdgcn_exp2f(sc[kk * GP + hh] - stat_m[hh]);
        sc[kk * GP + hh] = e;
        ls[hh] += e;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float s = ls[hh];
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s += __shfl_xor(s, 4);
      s += __shfl_xor(s, 8);
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (lane == 0) red[wave][hh] = s;
    }
  }
  __syncthreads();
  if (tid < G) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) s += red[w][tid];
    stat_l[tid] = s;
  }

  // ---- phase C: P.V ----
  {
    const int ksl = lane / LPV;   // key slot within the wavefront step
    const int dp = lane % LPV;    // 8-dim part
    float acc[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;

    for (int base = wave * KPW + ksl; base < cnt; base += NWAVES * KPW * UC) {
      u32x4 vr[UC];
#pragma unroll
      for (int u = 0; u < UC; ++u) {
        const int kk = base + NWAVES * KPW * u;
        if (kk < cnt) {
          const int key = sg.row(v0 + kk);
          vr[u] = ldg16_stream(vbase + (int64_t)key * p.vs_t + dp * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < UC; ++u) {
        const int kk = base + NWAVES * KPW * u;
        if (kk < cnt) {
          float vf[8];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            vf[2 * w] = bf_lo(vr[u][w]);
            vf[2 * w + 1] = bf_hi(vr[u][w]);
          }
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            const float pr = sc[kk * GP + hh];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[hh][e] = __builtin_fmaf(pr, vf[e], acc[hh][e]);
          }
        }
      }
    }
    // reduce over key slots (lanes dp, dp+LPV, ...)
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float a = acc[hh][e];
#pragma unroll
        for (int off = LPV; off < 64; off <<= 1) a += __shfl_xor(a, off);
        acc[hh][e] = a;
      }
    if (ksl == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        *reinterpret_cast<f32x4*>(&accs[wave][hh * D + dp * 8]) =
            f32x4{acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]};
        *reinterpret_cast<f32x4*>(&accs[wave][hh * D + dp * 8 + 4]) =
            f32x4{acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]};
      }
    }
  }
  __syncthreads();

  // ---- write this chunk's normalised output and log-sum-exp ----
  const int64_t pidx = ((int64_t)split * p.B + b) * p.Hq + (int64_t)h * G;
  for (int idx = tid; idx < G * D; idx += NTHREADS) {
    const int hh = idx / D;
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) a += accs[w][idx];
    p.opart[(pidx + hh) * D + (idx - hh * D)] = a / stat_l[hh];
  }
  if (tid < G) p.lsepart[pidx + tid] = (stat_m[tid] + __log2f(stat_l[tid])) * LN2;
}

// Merge of the chunks of one (sequence, query head) by log-sum-exp.  Four
// groups of 64 threads each sum a quarter of the chunks and are added in LDS.
// Up to 32 chunks, each group requests its chunks' outputs and log-sum-exps
// together and weights them once the maximum is known; beyond that the
// log-sum-exps are loaded one per thread first and the weights kept in LDS.
template <int D>
__global__ __launch_bounds__(NTHREADS) void cowa_decode_combine(DecodeParams p) {
  constexpr int MAXW = 1024;       // chunk weights held in LDS per pass
  constexpr int DPT = D / 64;      // dims per thread
  __shared__ float wts[MAXW];
  __shared__ float red[NWAVES];
  __shared__ __attribute__((aligned(16))) float part[NWAVES][D];
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int h = hq / p.G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int t;
  const Segs sg = decode_segs(p, b, h, &t);
  const int ns = (sg.total() + p.chunk - 1) / p.chunk;
  const int64_t stride_s = (int64_t)p.B * p.Hq;
  const int64_t base = (int64_t)b * p.Hq + hq;

  const float* op = p.opart + base * D + lane * DPT;
  float M;
  float o[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) o[i] = 0.f;
  float wsum = 0.f;   // summed over the wavefront below
  if (ns <= 4 * 8) {
    // At most eight chunks per group: the partial outputs and their
    // log-sum-exps are all requested before the maximum is known (one memory
    // round trip); every lane of a group holds the same eight weights.
    float v[8][DPT];
    float lw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = wave + 4 * u;
      lw[u] = NEG_INF;
      if (k < ns) {
        lw[u] = p.lsepart[k * stride_s + base];
#pragma unroll
        for (int i = 0; i < DPT; ++i) v[u][i] = op[(int64_t)k * stride_s * D + i];
      }
    }
    float m = NEG_INF;
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fmaxf(m, lw[u]);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float ws = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (wave + 4 * u < ns) {
        const float w = __expf(lw[u] - M);
        ws += w;
#pragma unroll
        for (int i = 0; i < DPT; ++i) o[i] = __builtin_fmaf(w, v[u][i], o[i]);
      }
    if (lane == 0) wsum = ws;
  } else {
    // maximum chunk log-sum-exp
    float m = NEG_INF;
    for (int s2 = tid; s2 < ns; s2 += NTHREADS) m = fmaxf(m, p.lsepart[s2 * stride_s + base]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();

    for (int s0 = 0; s0 < ns; s0 += MAXW) {
      const int nb = ns - s0 < MAXW ? ns - s0 : MAXW;
      for (int i = tid; i < nb; i += NTHREADS) {
        const float w = __expf(p.lsepart[(s0 + i) * stride_s + base] - M);
        wts[i] = w;
        wsum += w;
      }
      __syncthreads();
      // group `wave` takes chunks wave, wave + 4, ...
      int k = wave;
      for (; k + 4 * 7 < nb; k += 4 * 8) {
        float v[8][DPT];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int i = 0; i < DPT; ++i) v[u][i] = op[(int64_t)(s0 + k + 4 * u) * stride_s * D + i];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int i = 0; i < DPT; ++i) o[i] = __builtin_fmaf(wts[k + 4 * u], v[u][i], o[i]);
      }
      for (; k < nb; k += 4)
#pragma unroll
        for (int i = 0; i < DPT; ++i)
          o[i] = __builtin_fmaf(wts[k], op[(int64_t)(s0 + k) * stride_s * D + i], o[i]);
      __syncthreads();
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
  if (lane == 0) red[wave] = wsum;
#pragma unroll
  for (int i = 0; i < DPT; ++i) part[wave][lane * DPT + i] = o[i];
  __syncthreads();
  const float W = red[0] + red[1] + red[2] + red[3];
  if (wave == 0) {
    char* obase = reinterpret_cast<char*>(p.o);
    const int64_t oi = (int64_t)b * p.os_b + (int64_t)hq * p.os_h + lane * DPT;
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const int dd = lane * DPT + i;
      const float v = (part[0][dd] + part[1][dd] + part[2][dd] + part[3][dd]) / W;
      if (p.o_f32)
        reinterpret_cast<float*>(obase)[oi + i] = v;
      else
        reinterpret_cast<__bf16*>(obase)[oi + i] = (__bf16)v;
    }
    if (lane == 0) p.lse[base] = M + __logf(W);
  }
}

template <int D, int G>
void launch_split(const DecodeParams& p, hipStream_t s) {
  const dim3 grid((unsigned)p.n_splits, (unsigned)p.Hkv, (unsigned)p.B);
  hipLaunchKernelGGL((cowa_decode_split<D, G>), grid, dim3(NTHREADS), 0, s, p);
  hipLaunchKernelGGL((cowa_decode_combine<D>), dim3((unsigned)p.Hq, (unsigned)p.B),
                     dim3(NTHREADS), 0, s, p);
}

template <int D>
int dispatch_group(const DecodeParams& p, hipStream_t s) {
  switch (p.G) {
    case 1: launch_split<D, 1>(p, s); break;
    case 2: launch_split<D, 2>(p, s); break;
    case 3: launch_split<D, 3>(p, s); break;
    case 4: launch_split<D, 4>(p, s); break;
    case 5: launch_split<D, 5>(p, s); break;
    case 6: launch_split<D, 6>(p, s); break;
    case 7: launch_split<D, 7>(p, s); break;
    case 8: launch_split<D, 8>(p, s); break;
    default: return 1;
  }
  return 0;
}

}  // namespace

int launch_decode(const DecodeParams& p, int d, int o_f32, void* stream) {
  (void)o_f32;  // carried in p.o_f32
  hipStream_t s = static_cast<hipStream_t>(stream);
  int bad = d == 128 ? dispatch_group<128>(p, s) : dispatch_group<64>(p, s);
  if (bad) return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// Scratch of cowa_decode_noalloc: the split kernel's partial outputs and
// log-sum-exps, for callers that cannot allocate.  Every GPU holds its own
// copy at its own address; host code must use the address looked up below,
// never the symbol itself (in host code the symbol is only a stand-in).
static __device__ __align__(256) unsigned char scratch[COWA_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int decode_scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

}  // namespace cowa
