// gemm_mx.h -- one workgroup tile of an MXFP8 GEMM (E4M3 codes, one E8M0
// scale per 32 consecutive k of every operand row) on the CDNA4 scaled
// matrix-core instruction v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulate.
//
// A K stage is 128 bytes of every operand row -- 128 codes, where the bf16
// tile (gemm_bf16.h) stages 64 values -- so the LDS row layout (lds_idx), the
// KRows loader and the main loop are shared with the bf16 tile.  Each stage
// also carries the 4 scale codes of every row of both operands (one 32-bit
// word per row, k-blocks 0..3 of the stage in bytes 0..3): thread t loads
// the word of row t of [A rows | B rows] (BM + BN = 256 threads), and the
// words sit after the A codes of the stage.
//
// Operand layout of the instruction on gfx950 (checked with single-wave
// probes against an exact host product):
//   lane l feeds A row / B column l % 32; lane half h = l / 32 holds
//   k = 16h .. 16h+15 in bytes 0-15 of its 8 dwords and k = 32+16h ..
//   32+16h+15 in bytes 16-31, i.e. 16-byte chunks h and 2+h of the 64-byte
//   k range
//   the scale operand of lane l is the code of k-block h (k 32h .. 32h+31)
//   of that row / column, in the byte of the 32-bit register that the
//   op_sel argument names
//   the accumulator layout is the one of v_mfma_f32_32x32x16_bf16
// So for slice s (k 64s .. 64s+63) of a stage a lane reads chunks 4s+h and
// 4s+2+h of its row, and the scale of k-block 2s+h: byte 2s of the row's
// scale word shifted right by 8h.
#pragma once

#include <type_traits>

#include "gemm_bf16.h"

namespace moe {

template <int BM_, int BN_>
struct TileMX {
  static constexpr bool kMX = true;
  static constexpr bool kDMA = false;
  static constexpr bool kKeyHi = false;  // lds_key<false>
  static constexpr int BM = BM_, BN = BN_;
  static_assert(BM + BN == kThreads, "one scale row per thread");
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MI = WM / 32, NJ = WN / 32;
  // one stage, in bf16 units: A rows x 128 code bytes, then the scale words
  // of the A and B rows; B rows x 128 code bytes
  static constexpr int LDS_A = BM * 64 + (BM + BN) * 2, LDS_B = BN * 64;
  static constexpr size_t smem_bytes = 2 * (LDS_A + LDS_B) * sizeof(bf16_t);
  static_assert((LDS_A * sizeof(bf16_t)) % 16 == 0, "B stages stay 16-byte aligned");
  static __device__ __forceinline__ void stage(const bf16_t* As, const bf16_t* Bs, f32x16_t (&acc)[MI][NJ]);
};

// Codes of operand A (row-major [rows, K] bytes, k contiguous) through
// KRows, one 16-byte chunk of 16 codes per lane and row, plus the stage's
// scale word of row t of [A rows | B rows] for thread t (scale rows are
// [rows, K/32] bytes, 4-byte aligned).  Operand B's codes use KRows as is.
//
// A stage needs one scale word from each of 256 rows, 256 different lines.
// With wide rows (a multiple of 4 words, 16-byte aligned: K % 512 == 0)
// each thread reads its row's words of 4 consecutive stages at once, every
// fourth stage, so a scale line is touched a quarter as often and the
// expert weights streaming through the L2 between stages evict it less.
// The loads come in stage order from 0 (the main loop's order).
template <int ROWS, int BROWS>
struct KRowsMX {
  static_assert(ROWS + BROWS == kThreads, "one scale row per thread");
  KRows<ROWS> codes;
  const uint32_t* srow;
  uint32_t sv[kPrefetch];
  uint4 s4;   // words of stages 4g .. 4g+3 (wide rows)
  bool wide;
  // rowptr(r): first code byte of A row r; ascale(r), bscale(r): first
  // scale byte of A row r / B row r.  All must be readable for every row.
  template <class F, class GA, class GB>
  __device__ __forceinline__ void init(F rowptr, GA ascale, GB bscale, bool wide_rows) {
    codes.init([&](int r) { return (const bf16_t*)rowptr(r); });
    const int t = threadIdx.x;
    srow = t < ROWS ? (const uint32_t*)ascale(t) : (const uint32_t*)bscale(t - ROWS);
    wide = wide_rows;
  }
  __device__ __forceinline__ void prep(int) {}
  template <int BUF>
  __device__ __forceinline__ void load(int kt) {
    codes.template load<BUF>(kt);
    if (wide) {
      const int q = kt & 3;
      if (q == 0) s4 = *(const uint4*)(srow + kt);
      sv[BUF] = q == 0 ? s4.x : q == 1 ? s4.y : q == 2 ? s4.z : s4.w;
    } else {
      sv[BUF] = srow[kt];
    }
  }
  template <int BUF, bool HI>
  __device__ __forceinline__ void store(bf16_t* lds) const {
    static_assert(!HI, "the MX tile reads with lds_key<false>");
    codes.template store<BUF, HI>(lds);
    ((uint32_t*)(lds + ROWS * 64))[threadIdx.x] = sv[BUF];
  }
};

template <int OPSEL>
__device__ __forceinline__ f32x16_t mfma_mx(i32x8_t a, uint32_t sa, i32x8_t b, uint32_t sb, f32x16_t c) {
  // formats 0, 0: both operands E4M3
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, (int)sa, OPSEL, (int)sb);
}

// The 128-deep stage as 2 slices of 64: the fragments of both slices are
// read first (two 16-byte LDS reads per fragment and slice), then the MFMAs
// of slice 0 and of slice 1.
// sa, sb: the stage's scale words of the A rows and of the B rows.
template <class TL>
__device__ __forceinline__ void tile_compute_mx(const bf16_t* As, const bf16_t* Bs, const uint32_t* sa,
                                                const uint32_t* sb, f32x16_t (&acc)[TL::MI][TL::NJ]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, rr = lane & 31;
  auto frag = [&](const bf16_t* base, int row, int s) -> i32x8_t {
    const uint4 lo = *(const uint4*)(base + lds_idx<TL::kKeyHi>(row, 4 * s + h));
    const uint4 hi = *(const uint4*)(base + lds_idx<TL::kKeyHi>(row, 4 * s + 2 + h));
    i32x8_t v;
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    return v;
  };
  uint32_t xa[TL::MI], xb[TL::NJ];
#pragma unroll
  for (int i = 0; i < TL::MI; ++i) xa[i] = sa[wm * TL::WM + 32 * i + rr] >> (8 * h);
#pragma unroll
  for (int j = 0; j < TL::NJ; ++j) xb[j] = sb[wn * TL::WN + 32 * j + rr] >> (8 * h);
  auto slice = [&](auto opsel) {
    constexpr int s = decltype(opsel)::value;
    i32x8_t a[TL::MI], b[TL::NJ];
#pragma unroll
    for (int i = 0; i < TL::MI; ++i) a[i] = frag(As, wm * TL::WM + 32 * i + rr, s);
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j) b[j] = frag(Bs, wn * TL::WN + 32 * j + rr, s);
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
      for (int j = 0; j < TL::NJ; ++j) acc[i][j] = mfma_mx<2 * s>(a[i], xa[i], b[j], xb[j], acc[i][j]);
  };
  slice(std::integral_constant<int, 0>());
  slice(std::integral_constant<int, 1>());
}

template <int BM_, int BN_>
__device__ __forceinline__ void TileMX<BM_, BN_>::stage(const bf16_t* As, const bf16_t* Bs,
                                                       f32x16_t (&acc)[MI][NJ]) {
  const uint32_t* sa = (const uint32_t*)(As + BM * 64);
  tile_compute_mx<TileMX<BM_, BN_>>(As, Bs, sa, sa + BM, acc);
}

// ---------------------------------------------------------------- codec
// OCP Microscaling (MX) v1.0 MXFP8: E4M3 elements (bias 7, no infinity,
// largest finite 448) sharing an E8M0 scale 2^(code - 127) per block of 32.

// Scale code of a block whose largest magnitude is amax: the shared
// exponent floor(log2 amax) - 8 (8 = the largest E4M3 exponent), clamped
// below at -127, plus the bias 127.  The biased fp32 exponent of amax is
// floor(log2 amax) + 127 for normal amax; zero and subnormal amax give 0.
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return e > 8 ? (uint32_t)(e - 8) : 0u;
}

// 2^(127 - code) = 1 / scale, exactly (code <= 246, so the exponent field
// 254 - code stays in [8, 254]).
__device__ __forceinline__ float mx_inv_scale(uint32_t code) {
  return __uint_as_float((254u - code) << 23);
}

// Nearest-even E4M3 code of x (finite, |x| < 512 after scaling): the
// magnitude clamped to 448, its quantum 2^(e - 3) with e = max(floor(log2),
// -6) (the subnormal quantum 2^-9 below 2^-6), q = round-to-even(m /
// quantum) in [0, 16]; the code is 8 (e + 6) + q, which carries into the
// exponent field when q reaches 16.  Values that round to zero take code 0.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const float m = fminf(__uint_as_float(u & 0x7fffffffu), 448.0f);
  int e = (int)(__float_as_uint(m) >> 23) - 127;
  e = e < -6 ? -6 : e;
  const float q = __builtin_rintf(m * __uint_as_float((uint32_t)(130 - e) << 23));
  const uint32_t c = (uint32_t)((e + 6) * 8) + (uint32_t)q;
  return c ? (c | ((u >> 24) & 0x80u)) : 0u;
}

// One block of 32 values: the scale code and the 32 codes, 4 per word
// (value 4w + b in byte b of word w).
__device__ __forceinline__ uint32_t mx_quant32(const float (&v)[32], uint32_t (&w)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sc = mx_scale_code(amax);
  const float inv = mx_inv_scale(sc);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    w[q] = e4m3_code(v[4 * q] * inv) | (e4m3_code(v[4 * q + 1] * inv) << 8) |
           (e4m3_code(v[4 * q + 2] * inv) << 16) | (e4m3_code(v[4 * q + 3] * inv) << 24);
  return sc;
}

// Quantises 32 bf16 values at src: the 32 codes packed into w, the scale
// code returned.
__device__ __forceinline__ uint8_t mx_quant_bf16_words(const bf16_t* src, uint32_t (&w)[8]) {
  uint4 in[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) in[i] = ((const uint4*)src)[i];
  float v[32];
  const uint32_t* iw = (const uint32_t*)in;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = __uint_as_float(iw[i] << 16);
    v[2 * i + 1] = __uint_as_float(iw[i] & 0xffff0000u);
  }
  return (uint8_t)mx_quant32(v, w);
}

// Quantises block b of a bf16 row at src into codes (32 bytes at dst) and
// its scale code.
__device__ __forceinline__ void mx_quant_bf16_block(const bf16_t* src, uint8_t* dst, uint8_t* scale) {
  uint32_t w[8];
  *scale = mx_quant_bf16_words(src, w);
  ((uint4*)dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
  ((uint4*)dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

}  // namespace moe
