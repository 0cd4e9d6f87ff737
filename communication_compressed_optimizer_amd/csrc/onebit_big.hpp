// Kernels for chunks longer than 16384 elements (C = 4096 << lr, lr = 3..12,
// so chunks of 2^15 .. 2^24 elements; chunk length is a run-time value).
//
// A chunk is one workgroup of 256 threads that walks it in 4096-element
// blocks, each block in the slot layout of a 4096-element chunk of
// onebit_kernels.hpp (thread t owns slots t + 256k, k = 0..3).  Sign words
// need no change: element j of chunk k is bit (j mod 32) of word
// k*C/32 + j/32, so block b's 128 words follow those of block b - 1.
//
// Chunk scale.  The canonical sum of squares is the stride-halving tree
// over the chunk (h = C/2, ..., 1).  Its top lr levels pair, at every
// position p of a block, blocks b and b + R/2, then b and b + R/4, ...
// (R = 2^lr blocks): a pairwise tree over the blocks taken in bit-reversed
// order.  big_sumsq forms it block by block with a binary counter of
// partial trees per position (level L holds the sum over 2^L blocks) and
// then takes the 4096 per-position sums through the tree of a 4096-element
// chunk, so the result is the canonical tree bit for bit.  A block past
// the last valid element contributes +0.  The signs and errors need that
// scale, so a second walk over the blocks recomputes each block's values
// and compresses them.  Chunks of 2^15 and 2^16 elements (8 or 16 blocks)
// instead hold every block in registers (big_compress_res), form the same
// tree from them and compress from them, reading each input once.
//
// Per-(chunk, tensor) statistics (the rescale's maximum or double sums, the
// warmup's sums of x^2 and u^2) are formed block by block and combined by
// thread 0 in block order: the maximum does not depend on that order, and
// the double sums are reproducible and, in the warmup, the same in both
// passes, so a carried sum of x^2 is bit for bit the one pass 1 would form.
#pragma once

#include "onebit_kernels.hpp"

namespace onebit {

constexpr int kBlk = 4096;               // elements per block
constexpr int kBT = Geo<kBlk>::T;        // 256 threads per chunk
constexpr int kBigMinLog = 3;            // 2^15 elements: the first chunk longer than 16384
constexpr int kBigMaxLog = 12;           // 2^24 elements

// Chunk k of an n-element buffer in chunks of 4096 << lr elements.
struct BigAt {
  int64_t k, base, nk;  // chunk, its first element, its valid elements
  int lr;               // log2 of the blocks per chunk
  __device__ __forceinline__ BigAt(int64_t k_, int64_t n, int lr_) {
    k = k_;
    lr = lr_;
    const int64_t C = (int64_t)kBlk << lr;
    base = k * C;
    nk = n - base < C ? n - base : C;
  }
  __device__ __forceinline__ int blocks() const { return 1 << lr; }
  __device__ __forceinline__ int64_t bbase(int b) const { return base + (int64_t)b * kBlk; }
  // valid elements of block b (0 past the chunk's end)
  __device__ __forceinline__ int valid(int b) const {
    const int64_t v = nk - (int64_t)b * kBlk;
    return v <= 0 ? 0 : (v >= kBlk ? kBlk : (int)v);
  }
  // block b's sign words
  __device__ __forceinline__ int64_t word0(int b) const {
    return k * (((int64_t)kBlk << lr) / 32) + (int64_t)b * Geo<kBlk>::WORDS;
  }
};

template <bool NT>
__device__ __forceinline__ void bload(const float* __restrict__ p, const BigAt& ch, int b, int v,
                                      Slots& s) {
  if (v == kBlk) load_chunk<kBlk, false, NT>(p, ch.bbase(b), kBlk, s);
  else load_chunk<kBlk, true, NT>(p, ch.bbase(b), v, s);
}

template <bool NT>
__device__ __forceinline__ void bstore(float* __restrict__ p, const BigAt& ch, int b, int v,
                                       const Slots& s) {
  if (v == kBlk) store_chunk<kBlk, false, NT>(p, ch.bbase(b), kBlk, s);
  else store_chunk<kBlk, true, NT>(p, ch.bbase(b), v, s);
}

__device__ __forceinline__ void zero_slots(Slots& s) {
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) s[a][c] = 0.0f;
}

// Positions of a block past its v valid elements set to 0.
__device__ __forceinline__ void clear_past(Slots& s, int v) {
  if (v == kBlk) return;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (!slot_valid<kBlk>(a, c, v)) s[a][c] = 0.0f;
}

// The canonical sum of squares of chunk ch (see the file comment).  zf(b, v,
// z) gives block b's values (v valid, v > 0).
template <class ZF>
__device__ __forceinline__ float big_sumsq(const BigAt& ch, ZF&& zf, float4* lds, int& parity) {
  Slots st[kBigMaxLog + 1];
  const int R = ch.blocks();
  for (int i = 0; i < R; ++i) {
    const int b = (int)(__builtin_bitreverse32((uint32_t)i) >> (32 - ch.lr));
    Slots cur;
    const int v = ch.valid(b);
    if (v == 0) {
      zero_slots(cur);
    } else {
      zf(b, v, cur);
      clear_past(cur, v);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) cur[a][c] = cur[a][c] * cur[a][c];
    }
    // binary counter: the block enters at level 0; while bit L of i is set,
    // the partial tree of the 2^L blocks before it is its left operand
    bool carry = true;
#pragma unroll
    for (int L = 0; L <= kBigMaxLog; ++L) {
      if (carry) {
        if ((i >> L) & 1) {
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c) cur[a][c] = st[L][a][c] + cur[a][c];
        } else {
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c) st[L][a][c] = cur[a][c];
          carry = false;
        }
      }
    }
  }
  Slots tot;
#pragma unroll
  for (int L = 0; L <= kBigMaxLog; ++L)
    if (L == ch.lr) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) tot[a][c] = st[L][a][c];
    }
  return chunk_sumsq<kBlk, 4, false>(tot, lds, parity);
}

// Error-compensated compression of one block with the chunk's scale s (the
// second half of compress_slots): z becomes the error, nib the signs.
__device__ __forceinline__ void apply_scale(Slots& z, int v, float s, uint32_t (&nib)[4]) {
  clear_past(z, v);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t nb = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool b = z[k][c] >= 0.0f;
      nb |= (uint32_t)(b && (v == kBlk || slot_valid<kBlk>(k, c, v))) << c;
      z[k][c] = b ? z[k][c] - s : z[k][c] + s;
    }
    nib[k] = nb;
  }
}

// Both walks of an error-compensated compression of chunk ch: the scale
// from zf's values, then each block's signs (into words) and error (into
// err, may be NULL when nothing is stored).  The words of blocks past the
// chunk's end are written as 0.  Returns the scale.
template <bool NT, class ZF>
__device__ __forceinline__ float big_compress(const BigAt& ch, ZF&& zf, float* __restrict__ err,
                                              uint32_t* __restrict__ words, float4* lds,
                                              int& parity) {
  const float s = chunk_scale(big_sumsq(ch, zf, lds, parity), (int)ch.nk);
  for (int b = 0; b < ch.blocks(); ++b) {
    const int v = ch.valid(b);
    uint32_t nib[4] = {0u, 0u, 0u, 0u};
    if (v > 0) {
      Slots z;
      zf(b, v, z);
      apply_scale(z, v, s, nib);
      if (err) bstore<NT>(err, ch, b, v, z);
    }
    store_sign_words<kBlk>(words + ch.word0(b), nib);
  }
  return s;
}

// The same compression with the whole chunk held in registers (RES blocks
// of 16 values per thread, RES = 2^lr): zf is called once per block, so
// each input is read once.  With every block at hand, the top levels of the
// canonical tree are the stride-halving over the blocks themselves (block
// b with b + RES/2, then b + RES/4, ...), which is the order big_sumsq
// reaches through its bit-reversed walk.
// big_compress_held: the values already in z (positions past the chunk's
// end are cleared here).
template <int RES, bool NT>
__device__ __forceinline__ float big_compress_held(const BigAt& ch, Slots (&z)[RES],
                                                   float* __restrict__ err,
                                                   uint32_t* __restrict__ words, float4* lds,
                                                   int& parity) {
#pragma unroll
  for (int b = 0; b < RES; ++b) {
    const int v = ch.valid(b);
    if (v > 0) clear_past(z[b], v);
    else zero_slots(z[b]);
  }
  Slots t[RES / 2];
#pragma unroll
  for (int b = 0; b < RES / 2; ++b)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        t[b][a][c] = (z[b][a][c] * z[b][a][c]) + (z[b + RES / 2][a][c] * z[b + RES / 2][a][c]);
#pragma unroll
  for (int h = RES / 4; h >= 1; h /= 2)
#pragma unroll
    for (int b = 0; b < h; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) t[b][a][c] = t[b][a][c] + t[b + h][a][c];
  const float s = chunk_scale(chunk_sumsq<kBlk, 4, false>(t[0], lds, parity), (int)ch.nk);
#pragma unroll
  for (int b = 0; b < RES; ++b) {
    const int v = ch.valid(b);
    uint32_t nib[4] = {0u, 0u, 0u, 0u};
    if (v > 0) {
      apply_scale(z[b], v, s, nib);
      if (err) bstore<NT>(err, ch, b, v, z[b]);
    }
    store_sign_words<kBlk>(words + ch.word0(b), nib);
  }
  return s;
}

template <int RES, bool NT, class ZF>
__device__ __forceinline__ float big_compress_res(const BigAt& ch, ZF&& zf,
                                                  float* __restrict__ err,
                                                  uint32_t* __restrict__ words, float4* lds,
                                                  int& parity) {
  Slots z[RES];
#pragma unroll
  for (int b = 0; b < RES; ++b) {
    const int v = ch.valid(b);
    if (v > 0) zf(b, v, z[b]);
  }
  return big_compress_held<RES, NT>(ch, z, err, words, lds, parity);
}

// RES = 0: the two walks of big_compress; else the resident form.
template <int RES, bool NT, class ZF>
__device__ __forceinline__ float big_compress_any(const BigAt& ch, ZF&& zf, float* __restrict__ err,
                                                  uint32_t* __restrict__ words, float4* lds,
                                                  int& parity) {
  if constexpr (RES == 0) return big_compress<NT>(ch, zf, err, words, lds, parity);
  else return big_compress_res<RES, NT>(ch, zf, err, words, lds, parity);
}

// onebit_compress_ef: z = in + err
template <bool NT, int RES>
__global__ void __launch_bounds__(kBT, 1)
k_big_compress_ef(int64_t n, int lr, const float* __restrict__ in, float* __restrict__ err,
                  uint32_t* __restrict__ bits, float* __restrict__ scales, int32_t* status) {
  __shared__ float4 lds[2 * kBT];
  int parity = 0;
  const BigAt ch(blockIdx.x, n, lr);
  auto zf = [&](int b, int v, Slots& z) {
    Slots e;
    bload<NT>(in, ch, b, v, z);
    bload<NT>(err, ch, b, v, e);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) z[a][c] = z[a][c] + e[a][c];
  };
  const float s = big_compress_any<RES, NT>(ch, zf, err, bits, lds, parity);
  if (threadIdx.x == 0) {
    scales[ch.k] = s;
    if (!__builtin_isfinite(s)) flag(status, 1);
  }
}

// beta1*m for block b: from the fp32 momentum or (PM) from the previous
// server output (bits_m, scales_m).
template <bool NT, bool PM>
__device__ __forceinline__ void big_beta1_momentum(const BigAt& ch, int b, int v,
                                                   const float* __restrict__ m,
                                                   const uint32_t* __restrict__ bits_m,
                                                   const float* __restrict__ scales_m,
                                                   const Coef& cf, Slots& bm) {
  if constexpr (PM) {
    uint32_t pn[4];
    load_sign_nibbles<kBlk>(bits_m + ch.word0(b), pn);
    const float sp = scales_m[ch.k];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) bm[a][c] = cf.beta1 * signed_scale(pn, a, c, sp);
  } else {
    bload<NT>(m, ch, b, v, bm);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) bm[a][c] = cf.beta1 * bm[a][c];
  }
}

// One worker's chunk: z = (beta1*m + a1*g) + e compressed (NTM: the
// momentum read as streaming data too).
template <bool NT, bool NTM, bool PM, int RES>
__device__ __forceinline__ void big_worker_chunk(const BigAt& ch, const float* __restrict__ g,
                                                 float* __restrict__ e,
                                                 const float* __restrict__ m,
                                                 const uint32_t* __restrict__ bits_m,
                                                 const float* __restrict__ scales_m,
                                                 uint32_t* __restrict__ bits_w,
                                                 float* __restrict__ scales_w, const Coef& cf,
                                                 int32_t* status, float4* lds) {
  int parity = 0;
  auto zf = [&](int b, int v, Slots& z) {
    Slots gg, ee;
    big_beta1_momentum<NTM, PM>(ch, b, v, m, bits_m, scales_m, cf, z);
    bload<NT>(g, ch, b, v, gg);
    bload<NT>(e, ch, b, v, ee);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) z[a][c] = (z[a][c] + (cf.a1 * gg[a][c])) + ee[a][c];
  };
  const float s = big_compress_any<RES, NT>(ch, zf, e, bits_w, lds, parity);
  if (threadIdx.x == 0) {
    scales_w[ch.k] = s;
    if (!__builtin_isfinite(s)) flag(status, 1);
  }
}

// One worker: z = (beta1*m + a1*g) + e
template <bool NT, bool PM, int RES>
__global__ void __launch_bounds__(kBT, 1)
k_big_worker_compress(int64_t n, int lr, const float* __restrict__ g, float* __restrict__ e,
                      const float* __restrict__ m, const uint32_t* __restrict__ bits_m,
                      const float* __restrict__ scales_m, uint32_t* __restrict__ bits_w,
                      float* __restrict__ scales_w, Coef cf, int32_t* status) {
  __shared__ float4 lds[2 * kBT];
  big_worker_chunk<NT, NT, PM, RES>(BigAt(blockIdx.x, n, lr), g, e, m, bits_m, scales_m, bits_w,
                                    scales_w, cf, status, lds);
}

// All W workers in one launch (fp32 momentum), one workgroup per (chunk,
// worker).  Workgroup g takes chunk 8*((g/8)/W) + g mod 8 for worker
// (g/8) mod W, so the W workgroups of a chunk have the same g mod 8 (the
// same XCD, as workgroups are dealt to the eight XCDs in turn) and lie close
// in dispatch order: the momentum they share is then read from HBM once and
// from that XCD's L2 by the others, and so is read with ordinary (not
// streaming) loads.  Grid: ceil(K/8)*8*W workgroups; those past the last
// chunk return at once.
template <bool NT, int RES>
__global__ void __launch_bounds__(kBT, 1)
k_big_workers_compress(int64_t n, int lr, int W, Workers wk, const float* __restrict__ m,
                       Coef cf, int32_t* status) {
  __shared__ float4 lds[2 * kBT];
  const int64_t gi = blockIdx.x, r = gi >> 3;
  const int w = (int)(r % W);
  const int64_t k = (r / W) * 8 + (gi & 7);
  if (k * ((int64_t)kBlk << lr) >= n) return;
  big_worker_chunk<NT, false, false, RES>(BigAt(k, n, lr), wk.g[w], wk.e[w], m, nullptr, nullptr,
                                          wk.bits[w], wk.scales[w], cf, status, lds);
}

// The server: y = (mean of the W workers' +-s) + err_s, recompressed
template <bool NT, int RES>
__global__ void __launch_bounds__(kBT, 1)
k_big_average_packed(int64_t n, int lr, int W, PackedIn pin, float* __restrict__ err_s,
                     uint32_t* __restrict__ bits_out, float* __restrict__ scales_out,
                     int32_t* status) {
  __shared__ float4 lds[2 * kBT];
  int parity = 0;
  const BigAt ch(blockIdx.x, n, lr);
  const float fW = (float)W;
  // The workers in groups of kGrp: a group's sign words and scales are
  // loaded together, then added in worker order.  Holding 16 blocks leaves
  // no registers for a group (the compiler then moves the blocks to
  // scratch memory), so that form takes one worker at a time.
  constexpr int kGrp = RES == 16 ? 1 : 4;
  auto zf = [&](int b, int v, Slots& y) {
    Slots acc;
    for (int w0 = 0; w0 < W; w0 += kGrp) {
      float sg[kGrp];
      uint32_t nib[kGrp][4];
#pragma unroll
      for (int j = 0; j < kGrp; ++j)
        if (w0 + j < W) {
          sg[j] = pin.scales[w0 + j][ch.k];
          load_sign_nibbles<kBlk>(pin.bits[w0 + j] + ch.word0(b), nib[j]);
        }
#pragma unroll
      for (int j = 0; j < kGrp; ++j)
        if (w0 + j < W) {
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float sv = signed_scale(nib[j], a, c, sg[j]);
              acc[a][c] = w0 + j == 0 ? sv : acc[a][c] + sv;
            }
        }
    }
    bload<NT>(err_s, ch, b, v, y);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) y[a][c] = (acc[a][c] / fW) + y[a][c];
  };
  const float s = big_compress_any<RES, NT>(ch, zf, err_s, bits_out, lds, parity);
  if (threadIdx.x == 0) {
    scales_out[ch.k] = s;
    if (!__builtin_isfinite(s)) flag(status, 2);
  }
}

// onebit_decompress
template <bool NT>
__global__ void __launch_bounds__(kBT, 1)
k_big_decompress(int64_t n, int lr, const uint32_t* __restrict__ bits,
                 const float* __restrict__ scales, float* __restrict__ out) {
  const BigAt ch(blockIdx.x, n, lr);
  const float s = scales[ch.k];
  for (int b = 0; b < ch.blocks(); ++b) {
    const int v = ch.valid(b);
    if (v == 0) break;
    uint32_t nib[4];
    load_sign_nibbles<kBlk>(bits + ch.word0(b), nib);
    Slots o;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) o[a][c] = signed_scale(nib, a, c, s);
    bstore<NT>(out, ch, b, v, o);
  }
}

// 1-bit Adam update: x = x - lr*(mhat/(sqrt(v_frozen)+eta)), m = mhat
template <bool NT>
__global__ void __launch_bounds__(kBT, 1)
k_big_adam_update(int64_t n, int lr, const uint32_t* __restrict__ bits_s,
                  const float* __restrict__ scales_s, const float* __restrict__ v_frozen,
                  float* __restrict__ x, float* __restrict__ m, Coef cf) {
  const BigAt ch(blockIdx.x, n, lr);
  const float s2 = scales_s[ch.k];
  for (int b = 0; b < ch.blocks(); ++b) {
    const int v = ch.valid(b);
    if (v == 0) break;
    uint32_t nib[4];
    load_sign_nibbles<kBlk>(bits_s + ch.word0(b), nib);
    Slots xx, vz, mh;
    bload<NT>(x, ch, b, v, xx);
    bload<NT>(v_frozen, ch, b, v, vz);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        mh[a][c] = signed_scale(nib, a, c, s2);
        xx[a][c] = xx[a][c] - (cf.lr * (mh[a][c] / (__builtin_sqrtf(vz[a][c]) + cf.eta)));
      }
    bstore<NT>(x, ch, b, v, xx);
    if (m) bstore<NT>(m, ch, b, v, mh);
  }
}

// The tensors block b of chunk ch overlaps: [lb, le], starting the search at
// lb (the first tensor of the previous block, or the chunk's first).
__device__ __forceinline__ void block_tensors(const DevTable& tab, const BigAt& ch, int b, int v,
                                              int& lb, int& le) {
  const int64_t first = ch.bbase(b), last = first + v - 1;
  while (tab.off[lb + 1] <= first) ++lb;
  le = lb;
  while (tab.off[le + 1] <= last) ++le;
}

// The per-(chunk, tensor) maximum of q over block b's elements of tensors
// lb..le, combined into seg_max by thread 0 (the chunk's segments start at
// -inf).
__device__ __forceinline__ void big_segment_max(const DevTable& tab, const BigAt& ch, int b, int v,
                                                int lb, int le, const Slots& q, float* red,
                                                float* __restrict__ seg_max, int l0, int sb) {
  const int64_t base = ch.bbase(b);
  for (int l = lb; l <= le; ++l) {
    const int64_t lo = tab.off[l] - base, hi = tab.off[l + 1] - base;
    float mx = -__builtin_inff();
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * ((int)threadIdx.x + kBT * a) + c;
        if (j < v && j >= lo && j < hi) mx = max_nan(mx, q[a][c]);
      }
    mx = block_max<kBT>(mx, red);
    if (threadIdx.x == 0) seg_max[sb + (l - l0)] = max_nan(seg_max[sb + (l - l0)], mx);
  }
}

// The per-(chunk, tensor) double sums of a^2 and b^2 over block b, added by
// thread 0 to the running sums (HA / HB: which sums are formed).
template <bool HA, bool HB>
__device__ __forceinline__ void big_segment_sums(const DevTable& tab, const BigAt& ch, int b, int v,
                                                 int lb, int le, const Slots& a_, const Slots& b_,
                                                 double* red, double* __restrict__ seg_a,
                                                 double* __restrict__ seg_b, int l0, int sb) {
  const int64_t base = ch.bbase(b);
  for (int l = lb; l <= le; ++l) {
    const int64_t lo = tab.off[l] - base, hi = tab.off[l + 1] - base;
    double sa = 0.0, sb2 = 0.0;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * ((int)threadIdx.x + kBT * a) + c;
        if (j < v && j >= lo && j < hi) {
          if constexpr (HA) sa += (double)a_[a][c] * (double)a_[a][c];
          if constexpr (HB) sb2 += (double)b_[a][c] * (double)b_[a][c];
        }
      }
    block_sum2<kBT>(sa, sb2, red);
    if (threadIdx.x == 0) {
      if constexpr (HA) seg_a[sb + (l - l0)] += sa;
      if constexpr (HB) seg_b[sb + (l - l0)] += sb2;
    }
  }
}

// Thread 0 starts the chunk's segments: the maximum at -inf, sums at 0.
__device__ __forceinline__ void init_segments(const DevTable& tab, int64_t k, float* seg_max,
                                              double* seg_a, double* seg_b) {
  if (threadIdx.x == 0) {
    const int n = tab.l1[k] - tab.l0[k] + 1, sb = tab.seg[k];
    for (int i = 0; i < n; ++i) {
      if (seg_max) seg_max[sb + i] = -__builtin_inff();
      if (seg_a) seg_a[sb + i] = 0.0;
      if (seg_b) seg_b[sb + i] = 0.0;
    }
  }
}

// The receiver's statistics (rescale_stats_chunk, block by block)
template <bool NT, bool RN, bool PM>
__global__ void __launch_bounds__(kBT, 1)
k_big_rescale_stats(DevTable tab, int lr, const uint32_t* __restrict__ bits_s,
                    const float* __restrict__ scales_s, const float* __restrict__ m,
                    const uint32_t* __restrict__ bits_m, const float* __restrict__ scales_m,
                    const float* __restrict__ v_frozen, float* __restrict__ v_fresh,
                    float* __restrict__ seg_max, double* __restrict__ seg_z,
                    double* __restrict__ seg_f, Coef cf) {
  __shared__ float red[kBT / 64];
  __shared__ double dred[2 * (kBT / 64)];
  const BigAt ch(blockIdx.x, tab.N, lr);
  const int l0 = tab.l0[ch.k], sb = tab.seg[ch.k];
  if constexpr (RN) init_segments(tab, ch.k, nullptr, seg_z, seg_f);
  else init_segments(tab, ch.k, seg_max, nullptr, nullptr);
  const float s2 = scales_s[ch.k];
  int lb = l0, le = l0;
  for (int b = 0; b < ch.blocks(); ++b) {
    const int v = ch.valid(b);
    if (v == 0) break;
    uint32_t nib[4];
    load_sign_nibbles<kBlk>(bits_s + ch.word0(b), nib);
    Slots bm, vf, vz;
    big_beta1_momentum<NT, PM>(ch, b, v, m, bits_m, scales_m, cf, bm);
    bload<NT>(v_fresh, ch, b, v, vf);
    bload<NT>(v_frozen, ch, b, v, vz);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float mh = signed_scale(nib, a, c, s2);
        const float gh = (mh - bm[a][c]) / cf.a1;
        vf[a][c] = (cf.beta2 * vf[a][c]) + (cf.a2 * (gh * gh));
      }
    bstore<NT>(v_fresh, ch, b, v, vf);
    block_tensors(tab, ch, b, v, lb, le);
    if constexpr (RN) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          vz[a][c] = __builtin_sqrtf(vz[a][c]) + cf.eta;
          vf[a][c] = __builtin_sqrtf(vf[a][c]) + cf.eta;
        }
      big_segment_sums<true, true>(tab, ch, b, v, lb, le, vz, vf, dred, seg_z, seg_f, l0, sb);
    } else {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          vz[a][c] = (__builtin_sqrtf(vz[a][c]) + cf.eta) / (__builtin_sqrtf(vf[a][c]) + cf.eta);
      big_segment_max(tab, ch, b, v, lb, le, vz, red, seg_max, l0, sb);
    }
  }
}

// Per-element step sizes lr*c_l of block b (tensors lb..le).
__device__ __forceinline__ void big_step_sizes(const DevTable& tab, const BigAt& ch, int b, int lb,
                                               int le, const float* __restrict__ c_layer, float lr,
                                               Slots& st) {
  const float s0 = lr * c_layer[lb];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) st[a][c] = s0;
  if (lb != le) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t gi = ch.bbase(b) + 4 * ((int)threadIdx.x + kBT * a) + c;
        st[a][c] = lr * c_layer[tensor_of(tab, lb, le, gi)];
      }
  }
}

// Compression step, pass B (pass_b_chunk, block by block)
template <bool NT>
__global__ void __launch_bounds__(kBT, 1)
k_big_pass_b(DevTable tab, int lr, const uint32_t* __restrict__ bits_s,
             const float* __restrict__ scales_s, const float* __restrict__ v_frozen,
             float* __restrict__ x, float* __restrict__ m, const float* __restrict__ c_layer,
             Coef cf) {
  const BigAt ch(blockIdx.x, tab.N, lr);
  const float s = scales_s[ch.k];
  int lb = tab.l0[ch.k], le = lb;
  for (int b = 0; b < ch.blocks(); ++b) {
    const int v = ch.valid(b);
    if (v == 0) break;
    uint32_t nib[4];
    load_sign_nibbles<kBlk>(bits_s + ch.word0(b), nib);
    Slots vz, xx, mh, st;
    bload<NT>(v_frozen, ch, b, v, vz);
    bload<NT>(x, ch, b, v, xx);
    block_tensors(tab, ch, b, v, lb, le);
    big_step_sizes(tab, ch, b, lb, le, c_layer, cf.lr, st);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        mh[a][c] = signed_scale(nib, a, c, s);
        const float d = mh[a][c] / (__builtin_sqrtf(vz[a][c]) + cf.eta);
        xx[a][c] = cf.wd != 0.0f ? xx[a][c] - (st[a][c] * (d + (cf.wd * xx[a][c])))
                                 : xx[a][c] - (st[a][c] * d);
      }
    bstore<NT>(x, ch, b, v, xx);
    if (m) bstore<NT>(m, ch, b, v, mh);
  }
}

// Warmup pass 1 (warmup_pass1_chunk, block by block; XS: x^2 sums carried)
template <bool NT, bool XS>
__global__ void __launch_bounds__(kBT, 1)
k_big_warmup_pass1(DevTable tab, int lr, int W, Workers wk, const float* __restrict__ x,
                   float* __restrict__ m, float* __restrict__ v, double* __restrict__ seg_x,
                   double* __restrict__ seg_u, Coef cf) {
  __shared__ double red[2 * (kBT / 64)];
  const BigAt ch(blockIdx.x, tab.N, lr);
  const int l0 = tab.l0[ch.k], sb = tab.seg[ch.k];
  init_segments(tab, ch.k, nullptr, XS ? nullptr : seg_x, seg_u);
  const float fW = (float)W;
  int lb = l0, le = l0;
  for (int b = 0; b < ch.blocks(); ++b) {
    const int nv = ch.valid(b);
    if (nv == 0) break;
    Slots gs, mm, vv, u, xx;
    bload<NT>(wk.g[0], ch, b, nv, gs);
    for (int w = 1; w < W; ++w) {
      Slots g;
      bload<NT>(wk.g[w], ch, b, nv, g);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) gs[a][c] = gs[a][c] + g[a][c];
    }
    bload<NT>(m, ch, b, nv, mm);
    bload<NT>(v, ch, b, nv, vv);
    if constexpr (XS) zero_slots(xx);  // not read: weight decay is 0 here
    else bload<NT>(x, ch, b, nv, xx);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float gb = gs[a][c] / fW;
        mm[a][c] = (cf.beta1 * mm[a][c]) + (cf.a1 * gb);
        vv[a][c] = (cf.beta2 * vv[a][c]) + (cf.a2 * (gb * gb));
        u[a][c] = warmup_dir(mm[a][c], vv[a][c], xx[a][c], cf);
      }
    bstore<NT>(m, ch, b, nv, mm);
    bstore<NT>(v, ch, b, nv, vv);
    block_tensors(tab, ch, b, nv, lb, le);
    big_segment_sums<!XS, true>(tab, ch, b, nv, lb, le, xx, u, red, seg_x, seg_u, l0, sb);
  }
}

// Warmup pass 2 (warmup_pass2_chunk, block by block; XO: the updated x's
// sums of squares into x_sq, in pass 1's order)
template <bool NT, bool XO>
__global__ void __launch_bounds__(kBT, 1)
k_big_warmup_pass2(DevTable tab, int lr, const float* __restrict__ m, const float* __restrict__ v,
                   float* __restrict__ x, const float* __restrict__ c_layer,
                   double* __restrict__ x_sq, Coef cf) {
  __shared__ double red[2 * (kBT / 64)];
  const BigAt ch(blockIdx.x, tab.N, lr);
  const int l0 = tab.l0[ch.k], sb = tab.seg[ch.k];
  if constexpr (XO) init_segments(tab, ch.k, nullptr, x_sq, nullptr);
  int lb = l0, le = l0;
  for (int b = 0; b < ch.blocks(); ++b) {
    const int nv = ch.valid(b);
    if (nv == 0) break;
    Slots mm, vv, xx, st;
    bload<NT>(m, ch, b, nv, mm);
    bload<NT>(v, ch, b, nv, vv);
    bload<NT>(x, ch, b, nv, xx);
    block_tensors(tab, ch, b, nv, lb, le);
    big_step_sizes(tab, ch, b, lb, le, c_layer, cf.lr, st);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float u = warmup_dir(mm[a][c], vv[a][c], xx[a][c], cf);
        xx[a][c] = xx[a][c] - (st[a][c] * u);
      }
    bstore<NT>(x, ch, b, nv, xx);
    if constexpr (XO)
      big_segment_sums<true, false>(tab, ch, b, nv, lb, le, xx, xx, red, x_sq, nullptr, l0, sb);
  }
}

}  // namespace onebit
