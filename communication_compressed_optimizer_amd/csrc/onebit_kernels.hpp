// HIP kernels of the 1-bit LAMB step for gfx950 (CDNA4, 64-wide waves).
//
// Every kernel that touches chunks runs one workgroup per chunk of C
// elements with T = C/16 threads; thread t owns the four float4 slots
// p = t + T*k (k = 0..3) of its chunk, i.e. chunk elements 4p..4p+3.  The
// loads and stores of a wave are therefore 64 consecutive float4 (1 KiB) per
// slot: fully coalesced dwordx4 traffic.
//
// Chunk scale.  The sum of squares of a chunk is the stride-halving tree
// t[j] += t[j+h], h = C/2, ..., 1 (zero past the last valid element), which
// fixes one rounding order so that scales, and through error feedback every
// later sign, are reproducible bit for bit.  With the slot layout above the
// levels h >= 4 act on the float4 slot index p with strides P/2..1
// (P = C/4) independently per component; strides 2T and T pair a thread's
// own slots, strides T/2..64 pair waves (through LDS), strides 32..1 pair
// lanes (cross-lane shuffles), and the last two levels (h = 2, 1) combine
// the four components: (c0 + c2) + (c1 + c3).
//
// Packed signs.  Element 4p+c sits in word p/8 at bit 4(p mod 8)+c, so
// eight consecutive lanes each contribute one nibble to a word; three DPP
// OR steps (quad_perm 1032, quad_perm 2301, row_half_mirror) assemble the
// word in every lane of the group of eight and lane 8q stores it.
//
// All arithmetic that feeds a stored fp32 value is one IEEE operation per
// source operation: the file is compiled with contraction off, and division
// and square root are the correctly rounded ones.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace onebit {

constexpr int kMaxWorkers = 16;

// Hyper-parameters and their fp32-derived constants (computed on the host in
// fp32: a1 = 1-beta1, a2 = 1-beta2, kp = 1+kappa, km = 1-kappa).
struct Coef {
  float beta1, beta2, eta, lr, a1, a2, kp, km, c_min, c_max, f_min, f_max;
};

// Device view of the tensor table.
struct DevTable {
  const int64_t* off;   // [L+1] flat offset of each tensor
  const int32_t* l0;    // [K] first tensor touched by chunk k
  const int32_t* l1;    // [K] last tensor touched by chunk k
  const int32_t* seg;   // [K] index of segment (k, l0[k]); segment (k, l) = seg[k] + l - l0[k]
  const int32_t* lseg;  // [L+1] segments of tensor l are [lseg[l], lseg[l+1])
  int64_t N;
  int64_t K;
  int32_t L;
};

// Per-worker device pointers, passed by value in the kernel arguments.
struct Workers {
  const float* g[kMaxWorkers];
  float* e[kMaxWorkers];
  uint32_t* bits[kMaxWorkers];
  float* scales[kMaxWorkers];
};

struct PackedIn {
  const uint32_t* bits[kMaxWorkers];
  const float* scales[kMaxWorkers];
};

template <int C>
struct Geo {
  static_assert(C >= 1024 && C <= 16384 && (C & (C - 1)) == 0, "chunk must be 2^10..2^14");
  static constexpr int T = C / 16;      // threads per chunk
  static constexpr int NW = T / 64;     // waves per chunk
  static constexpr int WORDS = C / 32;  // sign words per chunk
};

using Slots = float[4][4];  // [slot k][component c]

// ---------------------------------------------------------------------------
// loads and stores of a chunk in the slot layout
// ---------------------------------------------------------------------------
template <int C>
__device__ __forceinline__ void load_chunk(const float* __restrict__ p, int64_t base, int nk,
                                           Slots& o) {
  constexpr int T = Geo<C>::T;
  const int t = threadIdx.x;
  if (nk == C) {
    const float4* q = reinterpret_cast<const float4*>(p + base);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 v = q[t + T * k];
      o[k][0] = v.x;
      o[k][1] = v.y;
      o[k][2] = v.z;
      o[k][3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * (t + T * k) + c;
        o[k][c] = j < nk ? p[base + j] : 0.0f;
      }
  }
}

template <int C>
__device__ __forceinline__ void store_chunk(float* __restrict__ p, int64_t base, int nk,
                                            const Slots& o) {
  constexpr int T = Geo<C>::T;
  const int t = threadIdx.x;
  if (nk == C) {
    float4* q = reinterpret_cast<float4*>(p + base);
#pragma unroll
    for (int k = 0; k < 4; ++k) q[t + T * k] = make_float4(o[k][0], o[k][1], o[k][2], o[k][3]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * (t + T * k) + c;
        if (j < nk) p[base + j] = o[k][c];
      }
  }
}

// ---------------------------------------------------------------------------
// canonical chunk sum of squares (see the header comment)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float uniform_f32(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// lds: 2*T float4 (double-buffered between consecutive calls, so one
// barrier per call suffices).  Returns the sum in every thread.
template <int C>
__device__ __forceinline__ float chunk_sumsq(const Slots& z, float4* __restrict__ lds, int& parity) {
  constexpr int T = Geo<C>::T;
  constexpr int NW = Geo<C>::NW;
  float p[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float q0 = z[0][c] * z[0][c];
    const float q1 = z[1][c] * z[1][c];
    const float q2 = z[2][c] * z[2][c];
    const float q3 = z[3][c] * z[3][c];
    p[c] = (q0 + q2) + (q1 + q3);  // slot strides 2T, then T
  }
  if constexpr (NW > 1) {
    float4* buf = lds + parity * T;
    parity ^= 1;
    buf[threadIdx.x] = make_float4(p[0], p[1], p[2], p[3]);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    float v[NW][4];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float4 a = buf[w * 64 + lane];
      v[w][0] = a.x;
      v[w][1] = a.y;
      v[w][2] = a.z;
      v[w][3] = a.w;
    }
#pragma unroll
    for (int h = NW / 2; h >= 1; h /= 2)
#pragma unroll
      for (int w = 0; w < h; ++w)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[w][c] = v[w][c] + v[w + h][c];  // thread strides T/2..64
#pragma unroll
    for (int c = 0; c < 4; ++c) p[c] = v[0][c];
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1)
#pragma unroll
    for (int c = 0; c < 4; ++c) p[c] = p[c] + __shfl_down(p[c], s, 64);  // lane strides 32..1
  return uniform_f32((p[0] + p[2]) + (p[1] + p[3]));                 // h = 2, then h = 1
}

__device__ __forceinline__ float chunk_scale(float S, int nk) {
  return __builtin_sqrtf(S) / __builtin_sqrtf((float)nk);
}

// ---------------------------------------------------------------------------
// sign words
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t or_group8(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  return x;
}

// nib[k]: bit c = sign of element 4(t+T*k)+c.  words: the chunk's C/32 words.
template <int C>
__device__ __forceinline__ void store_sign_words(uint32_t* __restrict__ words, const uint32_t (&nib)[4]) {
  constexpr int T = Geo<C>::T;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = or_group8(nib[k] << (4 * (t & 7)));
    if ((t & 7) == 0) words[(t + T * k) >> 3] = w;
  }
}

template <int C>
__device__ __forceinline__ void load_sign_nibbles(const uint32_t* __restrict__ words, uint32_t (&nib)[4]) {
  constexpr int T = Geo<C>::T;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) nib[k] = (words[(t + T * k) >> 3] >> (4 * (t & 7))) & 0xFu;
}

template <int C>
__device__ __forceinline__ bool slot_valid(int k, int c, int nk) {
  return 4 * ((int)threadIdx.x + Geo<C>::T * k) + c < nk;
}

// Error-compensated 1-bit compression of z in place (z becomes the error):
// returns s; nib receives the sign nibbles; sgn[k][c] = +-s.
// Slots past the last valid element are cleared first (they count as 0 in
// the chunk sum and their bits are 0).
template <int C>
__device__ __forceinline__ float compress_slots(Slots& z, int nk, float4* lds, int& parity,
                                                uint32_t (&nib)[4], Slots& sgn) {
  if (nk != C) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (!slot_valid<C>(k, c, nk)) z[k][c] = 0.0f;
  }
  const float s = chunk_scale(chunk_sumsq<C>(z, lds, parity), nk);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t nb = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool b = z[k][c] >= 0.0f;
      nb |= (uint32_t)(b && slot_valid<C>(k, c, nk)) << c;
      z[k][c] = b ? z[k][c] - s : z[k][c] + s;
      sgn[k][c] = b ? s : -s;
    }
    nib[k] = nb;
  }
  return s;
}

// ---------------------------------------------------------------------------
// block reductions for per-tensor statistics (fixed order: deterministic)
// ---------------------------------------------------------------------------
template <int T>
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, 64));
  if constexpr (T / 64 == 1) {
    return v;
  } else {
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < T / 64; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
  }
}

template <int T>
__device__ __forceinline__ void block_sum2(double& a, double& b, double* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    a += __shfl_xor(a, s, 64);
    b += __shfl_xor(b, s, 64);
  }
  if constexpr (T / 64 > 1) {
    if ((threadIdx.x & 63) == 0) {
      red[2 * (threadIdx.x >> 6)] = a;
      red[2 * (threadIdx.x >> 6) + 1] = b;
    }
    __syncthreads();
    a = red[0];
    b = red[1];
#pragma unroll
    for (int w = 1; w < T / 64; ++w) {
      a += red[2 * w];
      b += red[2 * w + 1];
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void flag(int32_t* status, int32_t bit) {
  if (status) atomicOr(status, bit);
}

// Tensor of the element at flat index gi within chunk k's tensor range.
__device__ __forceinline__ int tensor_of(const DevTable& tab, int l0, int l1, int64_t gi) {
  int l = l0;
  while (l < l1 && gi >= tab.off[l + 1]) ++l;
  return l;
}

// ===========================================================================
// kernels
// ===========================================================================

// onebit_compress_ef: z = in + err -> bits, scales, err
template <int C>
__global__ void __launch_bounds__(C / 16)
k_compress_ef(int64_t n, const float* __restrict__ in, float* __restrict__ err,
              uint32_t* __restrict__ bits, float* __restrict__ scales, int32_t* status) {
  __shared__ float4 lds[2 * Geo<C>::T];
  int parity = 0;
  const int64_t k = blockIdx.x;
  const int64_t base = k * C;
  const int nk = (int)min((int64_t)C, n - base);
  Slots z, e;
  load_chunk<C>(in, base, nk, z);
  load_chunk<C>(err, base, nk, e);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) z[a][c] = z[a][c] + e[a][c];
  uint32_t nib[4];
  Slots sgn;
  const float s = compress_slots<C>(z, nk, lds, parity, nib, sgn);
  store_chunk<C>(err, base, nk, z);
  store_sign_words<C>(bits + k * Geo<C>::WORDS, nib);
  if (threadIdx.x == 0) {
    scales[k] = s;
    if (!__builtin_isfinite(s)) flag(status, 1);
  }
}

// onebit_average_packed: y = mean of the workers' +-s, + err_s -> recompress
template <int C>
__global__ void __launch_bounds__(C / 16)
k_average_packed(int64_t n, int W, PackedIn pin, float* __restrict__ err_s,
                 uint32_t* __restrict__ bits_out, float* __restrict__ scales_out, int32_t* status) {
  __shared__ float4 lds[2 * Geo<C>::T];
  int parity = 0;
  const int64_t k = blockIdx.x;
  const int64_t base = k * C;
  const int nk = (int)min((int64_t)C, n - base);
  Slots acc, y;
  for (int w = 0; w < W; ++w) {
    const float s = pin.scales[w][k];
    uint32_t nib[4];
    load_sign_nibbles<C>(pin.bits[w] + k * Geo<C>::WORDS, nib);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float v = ((nib[a] >> c) & 1u) ? s : -s;
        acc[a][c] = w == 0 ? v : acc[a][c] + v;
      }
  }
  load_chunk<C>(err_s, base, nk, y);
  const float fW = (float)W;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) y[a][c] = (acc[a][c] / fW) + y[a][c];
  uint32_t nib[4];
  Slots sgn;
  const float s = compress_slots<C>(y, nk, lds, parity, nib, sgn);
  store_chunk<C>(err_s, base, nk, y);
  store_sign_words<C>(bits_out + k * Geo<C>::WORDS, nib);
  if (threadIdx.x == 0) {
    scales_out[k] = s;
    if (!__builtin_isfinite(s)) flag(status, 2);
  }
}

// onebit_decompress
template <int C>
__global__ void __launch_bounds__(C / 16)
k_decompress(int64_t n, const uint32_t* __restrict__ bits, const float* __restrict__ scales,
             float* __restrict__ out) {
  const int64_t k = blockIdx.x;
  const int64_t base = k * C;
  const int nk = (int)min((int64_t)C, n - base);
  const float s = scales[k];
  uint32_t nib[4];
  load_sign_nibbles<C>(bits + k * Geo<C>::WORDS, nib);
  Slots o;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) o[a][c] = ((nib[a] >> c) & 1u) ? s : -s;
  store_chunk<C>(out, base, nk, o);
}

// Compression step, pass A: every worker's momentum compression, the server
// average and recompression, the reconstructed gradient, the fresh variance
// and the per-(chunk, tensor) maximum of the rescale ratio.
template <int C>
__global__ void __launch_bounds__(C / 16)
k_compressed_pass_a(DevTable tab, int W, Workers wk, float* __restrict__ err_s,
                    const float* __restrict__ m, const float* __restrict__ v_frozen,
                    float* __restrict__ v_fresh, uint32_t* __restrict__ bits_s,
                    float* __restrict__ scales_s, float* __restrict__ seg_max, Coef cf,
                    int32_t* status) {
  constexpr int T = Geo<C>::T;
  __shared__ float4 lds[2 * T];
  __shared__ float red[T / 64];
  int parity = 0;
  const int64_t k = blockIdx.x;
  const int64_t base = k * C;
  const int nk = (int)min((int64_t)C, tab.N - base);

  Slots bm, acc;
  load_chunk<C>(m, base, nk, bm);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) bm[a][c] = cf.beta1 * bm[a][c];

  for (int w = 0; w < W; ++w) {
    Slots z, e;
    load_chunk<C>(wk.g[w], base, nk, z);
    load_chunk<C>(wk.e[w], base, nk, e);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) z[a][c] = (bm[a][c] + (cf.a1 * z[a][c])) + e[a][c];
    uint32_t nib[4];
    Slots sgn;
    const float s = compress_slots<C>(z, nk, lds, parity, nib, sgn);
    store_chunk<C>(wk.e[w], base, nk, z);
    if (wk.bits[w]) store_sign_words<C>(wk.bits[w] + k * Geo<C>::WORDS, nib);
    if (threadIdx.x == 0) {
      if (wk.scales[w]) wk.scales[w][k] = s;
      if (!__builtin_isfinite(s)) flag(status, 1);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[a][c] = w == 0 ? sgn[a][c] : acc[a][c] + sgn[a][c];
  }

  // server: average, add its error, recompress
  Slots y;
  load_chunk<C>(err_s, base, nk, y);
  const float fW = (float)W;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) y[a][c] = (acc[a][c] / fW) + y[a][c];
  uint32_t nib[4];
  Slots mhat;
  const float s2 = compress_slots<C>(y, nk, lds, parity, nib, mhat);
  store_chunk<C>(err_s, base, nk, y);
  store_sign_words<C>(bits_s + k * Geo<C>::WORDS, nib);
  if (threadIdx.x == 0) {
    scales_s[k] = s2;
    if (!__builtin_isfinite(s2)) flag(status, 2);
  }

  // reconstructed gradient, fresh variance, rescale ratio
  Slots vf, vz;
  load_chunk<C>(v_fresh, base, nk, vf);
  load_chunk<C>(v_frozen, base, nk, vz);
  Slots q;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float gh = (mhat[a][c] - bm[a][c]) / cf.a1;
      vf[a][c] = (cf.beta2 * vf[a][c]) + (cf.a2 * (gh * gh));
      q[a][c] = (__builtin_sqrtf(vz[a][c]) + cf.eta) / (__builtin_sqrtf(vf[a][c]) + cf.eta);
    }
  store_chunk<C>(v_fresh, base, nk, vf);

  const int l0 = tab.l0[k];
  const int l1 = tab.l1[k];
  const int sb = tab.seg[k];
  for (int l = l0; l <= l1; ++l) {
    const int64_t lo = tab.off[l] - base;
    const int64_t hi = tab.off[l + 1] - base;
    float mx = -__builtin_inff();
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * ((int)threadIdx.x + T * a) + c;
        if (j < nk && j >= lo && j < hi) mx = fmaxf(mx, q[a][c]);
      }
    mx = block_max<T>(mx, red);
    if (threadIdx.x == 0) seg_max[sb + (l - l0)] = mx;
  }
}

// Per tensor: rho = max of its segments, soft thresholds, c.
template <int TB>
__global__ void __launch_bounds__(TB)
k_rescale_finalize(DevTable tab, const float* __restrict__ seg_max, const float* __restrict__ c_avg,
                   float* __restrict__ f_prev, float* __restrict__ c_layer, float* __restrict__ c_out,
                   Coef cf, int32_t* status) {
  __shared__ float red[TB / 64];
  const int l = blockIdx.x;
  const int lo = tab.lseg[l];
  const int hi = tab.lseg[l + 1];
  float mx = -__builtin_inff();
  for (int i = lo + (int)threadIdx.x; i < hi; i += TB) mx = fmaxf(mx, seg_max[i]);
  mx = block_max<TB>(mx, red);
  if (threadIdx.x == 0) {
    const float fp = f_prev[l];
    float f = fminf(fminf(mx, cf.f_max), cf.kp * fp);
    f = fmaxf(fmaxf(f, cf.f_min), cf.km * fp);
    f_prev[l] = f;
    const float c = c_avg[l] * f;
    c_layer[l] = c;
    if (c_out) c_out[l] = c;
    if (!__builtin_isfinite(mx)) flag(status, 8);
  }
}

// Compression step, pass B: x update with the per-tensor c, m = mhat.
template <int C>
__global__ void __launch_bounds__(C / 16)
k_compressed_pass_b(DevTable tab, const uint32_t* __restrict__ bits_s,
                    const float* __restrict__ scales_s, const float* __restrict__ v_frozen,
                    float* __restrict__ x, float* __restrict__ m, const float* __restrict__ c_layer,
                    Coef cf) {
  constexpr int T = Geo<C>::T;
  const int64_t k = blockIdx.x;
  const int64_t base = k * C;
  const int nk = (int)min((int64_t)C, tab.N - base);
  const float s = scales_s[k];
  uint32_t nib[4];
  load_sign_nibbles<C>(bits_s + k * Geo<C>::WORDS, nib);
  Slots vz, xx, mh;
  load_chunk<C>(v_frozen, base, nk, vz);
  load_chunk<C>(x, base, nk, xx);
  const int l0 = tab.l0[k];
  const int l1 = tab.l1[k];
  const float step0 = cf.lr * c_layer[l0];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float step = step0;
      if (l0 != l1) {
        const int64_t gi = base + 4 * ((int)threadIdx.x + T * a) + c;
        step = cf.lr * c_layer[tensor_of(tab, l0, l1, gi)];
      }
      mh[a][c] = ((nib[a] >> c) & 1u) ? s : -s;
      xx[a][c] = xx[a][c] - (step * (mh[a][c] / (__builtin_sqrtf(vz[a][c]) + cf.eta)));
    }
  store_chunk<C>(x, base, nk, xx);
  store_chunk<C>(m, base, nk, mh);
}

// Warmup pass 1: mean gradient, moments, per-(chunk, tensor) sums of x^2 and
// u^2 in double.
template <int C>
__global__ void __launch_bounds__(C / 16)
k_warmup_pass1(DevTable tab, int W, Workers wk, const float* __restrict__ x, float* __restrict__ m,
               float* __restrict__ v, double* __restrict__ seg_x, double* __restrict__ seg_u,
               Coef cf) {
  constexpr int T = Geo<C>::T;
  __shared__ double red[2 * (T / 64)];
  const int64_t k = blockIdx.x;
  const int64_t base = k * C;
  const int nk = (int)min((int64_t)C, tab.N - base);
  Slots gs;
  load_chunk<C>(wk.g[0], base, nk, gs);
  for (int w = 1; w < W; ++w) {
    Slots g;
    load_chunk<C>(wk.g[w], base, nk, g);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) gs[a][c] = gs[a][c] + g[a][c];
  }
  Slots mm, vv, u;
  load_chunk<C>(m, base, nk, mm);
  load_chunk<C>(v, base, nk, vv);
  const float fW = (float)W;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float gb = gs[a][c] / fW;
      mm[a][c] = (cf.beta1 * mm[a][c]) + (cf.a1 * gb);
      vv[a][c] = (cf.beta2 * vv[a][c]) + (cf.a2 * (gb * gb));
      u[a][c] = mm[a][c] / (__builtin_sqrtf(vv[a][c]) + cf.eta);
    }
  store_chunk<C>(m, base, nk, mm);
  store_chunk<C>(v, base, nk, vv);
  Slots xx;
  load_chunk<C>(x, base, nk, xx);
  const int l0 = tab.l0[k];
  const int l1 = tab.l1[k];
  const int sb = tab.seg[k];
  for (int l = l0; l <= l1; ++l) {
    const int64_t lo = tab.off[l] - base;
    const int64_t hi = tab.off[l + 1] - base;
    double sx = 0.0, su = 0.0;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * ((int)threadIdx.x + T * a) + c;
        if (j < nk && j >= lo && j < hi) {
          sx += (double)xx[a][c] * (double)xx[a][c];
          su += (double)u[a][c] * (double)u[a][c];
        }
      }
    block_sum2<T>(sx, su, red);
    if (threadIdx.x == 0) {
      seg_x[sb + (l - l0)] = sx;
      seg_u[sb + (l - l0)] = su;
    }
  }
}

// Per tensor: norms, trust ratio, clip, c_sum.
template <int TB>
__global__ void __launch_bounds__(TB)
k_warmup_finalize(DevTable tab, const double* __restrict__ seg_x, const double* __restrict__ seg_u,
                  float* __restrict__ c_sum, float* __restrict__ c_layer, float* __restrict__ c_out,
                  Coef cf, int32_t* status) {
  __shared__ double red[2 * (TB / 64)];
  const int l = blockIdx.x;
  const int lo = tab.lseg[l];
  const int hi = tab.lseg[l + 1];
  double X = 0.0, U = 0.0;
  for (int i = lo + (int)threadIdx.x; i < hi; i += TB) {
    X += seg_x[i];
    U += seg_u[i];
  }
  block_sum2<TB>(X, U, red);
  if (threadIdx.x == 0) {
    const float r = (X == 0.0 || U == 0.0) ? 1.0f : (float)(__builtin_sqrt(X) / __builtin_sqrt(U));
    const float c = fminf(fmaxf(r, cf.c_min), cf.c_max);
    c_sum[l] = c_sum[l] + c;
    c_layer[l] = c;
    if (c_out) c_out[l] = c;
    if (!__builtin_isfinite(X) || !__builtin_isfinite(U)) flag(status, 4);
  }
}

// Warmup pass 2: x = x - (lr*c_l)*u with u recomputed from the new m, v.
template <int C>
__global__ void __launch_bounds__(C / 16)
k_warmup_pass2(DevTable tab, const float* __restrict__ m, const float* __restrict__ v,
               float* __restrict__ x, const float* __restrict__ c_layer, Coef cf) {
  constexpr int T = Geo<C>::T;
  const int64_t k = blockIdx.x;
  const int64_t base = k * C;
  const int nk = (int)min((int64_t)C, tab.N - base);
  Slots mm, vv, xx;
  load_chunk<C>(m, base, nk, mm);
  load_chunk<C>(v, base, nk, vv);
  load_chunk<C>(x, base, nk, xx);
  const int l0 = tab.l0[k];
  const int l1 = tab.l1[k];
  const float step0 = cf.lr * c_layer[l0];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float step = step0;
      if (l0 != l1) {
        const int64_t gi = base + 4 * ((int)threadIdx.x + T * a) + c;
        step = cf.lr * c_layer[tensor_of(tab, l0, l1, gi)];
      }
      const float u = mm[a][c] / (__builtin_sqrtf(vv[a][c]) + cf.eta);
      xx[a][c] = xx[a][c] - (step * u);
    }
  store_chunk<C>(x, base, nk, xx);
}

// Freeze, element part: v_fresh = v, error buffers cleared.
template <int C>
__global__ void __launch_bounds__(C / 16)
k_freeze_elems(int64_t n, int W, const float* __restrict__ v, float* __restrict__ v_fresh,
               Workers wk, float* __restrict__ err_s) {
  const int64_t k = blockIdx.x;
  const int64_t base = k * C;
  const int nk = (int)min((int64_t)C, n - base);
  Slots vv, zero;
  load_chunk<C>(v, base, nk, vv);
  store_chunk<C>(v_fresh, base, nk, vv);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) zero[a][c] = 0.0f;
  for (int w = 0; w < W; ++w) store_chunk<C>(wk.e[w], base, nk, zero);
  store_chunk<C>(err_s, base, nk, zero);
}

// Freeze, tensor part: c_avg = c_sum / T_w, f_prev = 1.
__global__ void __launch_bounds__(256)
k_freeze_tensors(int L, const float* __restrict__ c_sum, float Tw, float* __restrict__ c_avg,
                 float* __restrict__ f_prev) {
  const int l = blockIdx.x * 256 + threadIdx.x;
  if (l < L) {
    c_avg[l] = c_sum[l] / Tw;
    f_prev[l] = 1.0f;
  }
}

}  // namespace onebit
