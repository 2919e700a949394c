// Paged decode attention and KV append for MI355X (gfx950, CDNA4).
//
// What is computed: for sequence b and query head h, the newest query scores
// every cached key of KV head h / g (g = Hq / Hkv), the scaled scores pass
// through a softmax, and the output is the weighted sum of the cached values
// (§1.1 of "The KV Cache Problem of Traditional Attention", pyllm.pages.dev;
// §1.2 and §2.2 of "Understanding KV Cache", steinslab.io). K/V are gathered
// through the block table (page "KV Cache and Inference Optimization",
// section "PagedAttention"; slot rule of "Understanding KV Cache" §3.3).
//
// Work decomposition: one wavefront per
//   (sequence b, KV head j, head group hg, context partition p),
// up to four such waves (consecutive KV heads) per workgroup.
// A partition is `pb_per_part` consecutive 16-token blocks of one sequence;
// the wave streams them once, so each K/V byte is read from HBM exactly once
// for the whole GQA group. Up to 16 query heads of the group form the N (or M)
// side of 16x16 MFMA tiles:
//
//   scores  S^T[t, h] = K[t, :] . Q[h, :]        MFMA, A = K tile (16 tokens),
//                                                B = Q^T (16 heads)
//   output  O^T[d, h] += V^T[d, t] P^T[t, h]     MFMA, A = V^T, B = P^T
//
// Register layouts (verified on gfx950 for every MFMA used here): lane
// l = 16 * q4 + r supplies A[row r][k-slots of quarter q4] and
// B[k-slots of quarter q4][col r]; result element i of lane l is D[4*q4 + i][r].
//  * K: lane (q4, r) loads token r's 16-byte chunks 4c + q4 -- exactly the A
//    operand, and Q's B operand uses the same d permutation.
//  * V: lane (q4, r) loads rows 4*q4 + i (i = 0..3), bytes [r*E, r*E + E)
//    (E = D/16 elements), i.e. each quarter-wave reads whole 256-byte rows.
//    Relabelling the output rows as d = r*E + mt makes these registers the
//    A operand of M-tile mt after packing 16-bit halves; no LDS transpose.
//  * The score tile's lane (q4, h) holds tokens 4*q4 + i for head h: exactly
//    the B operand P^T of the PV product, so P never moves between lanes.
//  * Output lane (q4, h) holds d = (4*q4 + i) * E + mt: 4E contiguous values.
// Softmax is online per head (running max m and sum l, log2 domain), with
// the maxima shared by the four lanes of a head through two cross-row lane
// swaps (v_permlane32_swap, v_permlane16_swap).
// For 16-bit inputs the weights enter the PV MFMA as a 16-bit head plus a
// 16-bit residual: rounding them once to bf16 would cost ~2^-9 relative per
// weight, enough to break a 2e-3 absolute bound on short contexts.
//
// When a sequence has several partitions, each writes o_p = acc / l and
// lse_p = m + log2(l) (fp32) and a merge kernel combines them:
// out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M), M = max_p lse_p.
#include <hip/hip_runtime.h>
#include <pkv.h>
#include <stdint.h>

#include <array>
#include <mutex>

namespace {

using f32x4 = float __attribute__((ext_vector_type(4)));
using u32x4 = unsigned __attribute__((ext_vector_type(4)));
using u32x2 = unsigned __attribute__((ext_vector_type(2)));
using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using f16x8 = _Float16 __attribute__((ext_vector_type(8)));
using s16x4 = short __attribute__((ext_vector_type(4)));
using f16x4 = _Float16 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;  // token rows per MFMA tile; a cache block holds block_size / 16 tiles
// 16-row tiles per partition of the decode, stream and one-wave prefill
// kernels: two tile addresses per lane
constexpr int kMaxPartitionBlocks = 128;
// 16-row tiles per partition of the LDS prefill kernel, whose partition's
// tile rows sit in an LDS table (4 bytes a tile)
#ifndef PKV_PREFILL_MAX_TILES
#define PKV_PREFILL_MAX_TILES 1024
#endif
constexpr int kMaxPrefillTiles = PKV_PREFILL_MAX_TILES;

// K/V blocks kept in flight per wave ahead of the one being consumed
#ifndef PKV_AHEAD_16BIT
#define PKV_AHEAD_16BIT 2
#endif
#ifndef PKV_AHEAD_32BIT
#define PKV_AHEAD_32BIT 1
#endif
#ifndef PKV_AHEAD_FP8
#define PKV_AHEAD_FP8 2
#endif
#ifndef PKV_XCD_ROTATE
#define PKV_XCD_ROTATE 1
#endif
#ifndef PKV_PARTITION_TARGET
#define PKV_PARTITION_TARGET 512
#endif
#ifndef PKV_DECODE_PAIRS
#define PKV_DECODE_PAIRS 1
#endif
#ifndef PKV_PREFILL_PAIRS
#define PKV_PREFILL_PAIRS 1
#endif
#ifndef PKV_AHEAD_PREFILL
#define PKV_AHEAD_PREFILL 2
#endif
#ifndef PKV_PAIR_RING  // tile pairs held in the register ring (16-bit caches)
#define PKV_PAIR_RING 2
#endif
#ifndef PKV_PAIR_RING_8BIT  // the same for 8-bit caches
#define PKV_PAIR_RING_8BIT 2
#endif
#ifndef PKV_KRING_8BIT  // 8-bit K of head size 128 (HND) through a per-wave LDS ring
#define PKV_KRING_8BIT 1
#endif
// bytes of that ring per wave: the ring's tiles of 16 rows x 128 codes
constexpr size_t kKRingWaveBytes = size_t(2) * PKV_PAIR_RING_8BIT * 16 * 128;
#ifndef PKV_RING_ROTATIONS
#define PKV_RING_ROTATIONS 3
#endif
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;  // weights are kept <= 2^8 between rescales

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor_shuffle(float v, int mask) {
  const int lane = static_cast<int>(__lane_id());
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

using lds_void = __attribute__((address_space(3))) void;
using s16x4_t = short __attribute__((ext_vector_type(4)));
using lds_s16x4 = __attribute__((address_space(3))) s16x4_t;
using i32x2_t = int __attribute__((ext_vector_type(2)));
using lds_i32x2 = __attribute__((address_space(3))) i32x2_t;
__device__ __forceinline__ lds_void* lds_ptr(char* p) { return (lds_void*)(p); }

// IEEE maximum (a NaN operand gives NaN): unlike fmaxf it needs no operand
// canonicalisation, and three-operand forms exist (v_maximum3_f32)
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four quarters of
// the wave) with gfx950's cross-row swaps: no LDS round trip
__device__ __forceinline__ float quarter_max(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmax_nan(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_nan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// the maximum over the four lanes of a score column (the decode kernel's
// quarter-waves), by permlane swaps or, for comparison, two LDS shuffles
#ifndef PKV_PERMLANE_MAX
#define PKV_PERMLANE_MAX 1
#endif
__device__ __forceinline__ float row_max4(float x) {
  if (PKV_PERMLANE_MAX) return quarter_max(x);
  x = fmaxf(x, xor_shuffle(x, 16));
  return fmaxf(x, xor_shuffle(x, 32));
}

// float -> 16-bit storage, round to nearest even; returns the bits
template <typename T>
__device__ __forceinline__ unsigned to_bits16(float x);
template <>
__device__ __forceinline__ unsigned to_bits16<__bf16>(float x) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(x));
}
template <>
__device__ __forceinline__ unsigned to_bits16<_Float16>(float x) {
  return __builtin_bit_cast(unsigned short, static_cast<_Float16>(x));
}
template <typename T>
__device__ __forceinline__ float from_bits16(unsigned b);
template <>
__device__ __forceinline__ float from_bits16<__bf16>(unsigned b) {
  return __uint_as_float(b << 16);
}
template <>
__device__ __forceinline__ float from_bits16<_Float16>(unsigned b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(b)));
}

// Two weights as a packed 16-bit head (hi) and the packed 16-bit rounding of
// what the head leaves out (lo): hi + lo carries about 16 significant bits.
// Any rounding of the head works (the residual is exact in fp32), so fp16
// uses the packed round-toward-zero conversion.
using f32x2 = float __attribute__((ext_vector_type(2)));
using bf16x2 = __bf16 __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ void split16_pair(float p0, float p1, unsigned& hi, unsigned& lo);
template <>
__device__ __forceinline__ void split16_pair<__bf16>(float p0, float p1, unsigned& hi, unsigned& lo) {
  hi = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{p0, p1}, bf16x2));
  const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{p0 - h0, p1 - h1}, bf16x2));
}
template <>
__device__ __forceinline__ void split16_pair<_Float16>(float p0, float p1, unsigned& hi, unsigned& lo) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(p0, p1);
  hi = __builtin_bit_cast(unsigned, h);
  lo = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(p0 - static_cast<float>(h[0]),
                                                                p1 - static_cast<float>(h[1])));
}

// Two floats that T represents exactly -> one packed dword (first value in
// the low half), with one packed conversion (the rounding mode is moot).
template <typename T>
__device__ __forceinline__ unsigned pack16_exact(float a, float b);
template <>
__device__ __forceinline__ unsigned pack16_exact<__bf16>(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
template <>
__device__ __forceinline__ unsigned pack16_exact<_Float16>(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// one QK MFMA step on a 16-byte chunk (16-bit types: 8 elements)
template <typename T>
__device__ __forceinline__ f32x4 mfma_qk16(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma_qk16<__bf16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                  0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_qk16<_Float16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                 0);
}
// one PV MFMA step (16-bit types: 4 tokens per lane)
template <typename T>
__device__ __forceinline__ f32x4 mfma_pv16(u32x2 a, u32x2 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma_pv16<__bf16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                    0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_pv16<_Float16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                                0);
}

// K/V tiles are read through buffer resources whose record count covers only
// the tile's valid rows: rows past the sequence end (NaN padding) and whole
// blocks past the partition end read as zeros with no memory traffic, so the
// load stream needs no branches. The loads carry the nontemporal hint: K/V are
// read exactly once per step, and streaming them without cache allocation
// measured ~6.9 TB/s vs ~6.1 TB/s for plain loads (permuted 4 KiB tiles).
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer format (gfx9 family)
constexpr int kCacheNT = 2;               // nontemporal cache policy
constexpr int kCacheDeviceCoherent = 16;  // sc1: coherent across XCDs (written through / read past the L2)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), static_cast<short>(0), bytes, kBufferWord3);
}

template <int NDW>
__device__ __forceinline__ void load_dwords(unsigned (&dst)[NDW], __amdgpu_buffer_rsrc_t rs, int off) {
  if constexpr (NDW == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kCacheNT);
    dst[0] = v[0];
    dst[1] = v[1];
  } else {
    static_assert(NDW % 4 == 0, "row slice must be 8 bytes or a multiple of 16");
#pragma unroll
    for (int w = 0; w < NDW; w += 4) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + w * 4, 0, kCacheNT);
      dst[w] = v[0];
      dst[w + 1] = v[1];
      dst[w + 2] = v[2];
      dst[w + 3] = v[3];
    }
  }
}

template <int NDW>
__device__ __forceinline__ void store_dwords(char* dst, const unsigned (&src)[NDW]) {
  if constexpr (NDW == 2) {
    *reinterpret_cast<u32x2*>(dst) = u32x2{src[0], src[1]};
  } else {
#pragma unroll
    for (int w = 0; w < NDW; w += 4)
      *reinterpret_cast<u32x4*>(dst + w * 4) = u32x4{src[w], src[w + 1], src[w + 2], src[w + 3]};
  }
}

// ---------------------------------------------------------------------------
// per-(T, D) constants
// ---------------------------------------------------------------------------
template <typename T, int D>
struct Shape {
  static constexpr int kElt = sizeof(T);
  static constexpr int kRowBytes = D * kElt;     // one token of one KV head
  static constexpr int kNK = kRowBytes / 64;     // 16-byte K chunks per lane
  static constexpr int kE = D / 16;              // V elements per lane per row
  static constexpr int kVDW = kE * kElt / 4;     // V dwords per lane per row
  static_assert(kRowBytes % 64 == 0, "head row must split into 4 x 16-byte chunk groups");
};

template <typename T, int D>
struct BlockRegs {
  u32x4 k[Shape<T, D>::kNK];
  unsigned v[4][Shape<T, D>::kVDW];
};

// Load one 16-row tile of K (MFMA A-operand layout) and V (row layout); token
// row r of the tile starts r * rs bytes after kt / vt (rs = the row bytes for
// HND caches, num_kv_heads times that for NHD). Only the first `rows` rows are
// fetched (the buffer bound is rows * rs), the rest read as zero.
template <typename T, int D>
__device__ __forceinline__ void load_block(BlockRegs<T, D>& r, const char* kt, const char* vt, int rows, int q4,
                                           int ln, int rs) {
  using S = Shape<T, D>;
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kt, rows * rs);
  const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vt, rows * rs);
#pragma unroll
  for (int c = 0; c < S::kNK; ++c) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, ln * rs + (4 * c + q4) * 16, 0, kCacheNT);
    r.k[c] = u32x4{v[0], v[1], v[2], v[3]};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) load_dwords<S::kVDW>(r.v[i], rv, (4 * q4 + i) * rs + ln * S::kE * S::kElt);
}

// ---------------------------------------------------------------------------
// FP8 (OCP E4M3) caches: one code byte per element plus one fp32 scale per
// token row of one KV head; the value attended over is code * scale.
// ---------------------------------------------------------------------------
// Raw registers of one FP8 block. K: lane (q4, r) holds token r's 16-byte
// chunks q4 + 4c (c < D/64), so each load instruction reads 64 contiguous
// bytes of every row (scattered 16-byte pieces per instruction cost a
// measured 5% of the stream rate); MFMA chunk c is bytes 8c..8c+7 of the
// lane's chunks taken in order, and the queries use the same d order
// (k_slice_elt). V: rows 4*q4 + i, bytes [r*D/16, r*D/16 + D/16).
// ks / vs: the scales of rows 4*q4 + i.
template <int D>
struct Fp8Regs {
  u32x4 k[D / 64];
  unsigned v[4][D / 64];
  f32x4 ks, vs;
};
// element index (d) of the e-th K code a lane (q4, r) holds: chunk q4 + 4 (e / 16), byte e % 16
template <int D>
__device__ __forceinline__ int k_slice_elt(int q4, int e) {
  return (q4 + 4 * (e >> 4)) * 16 + (e & 15);
}

// rs: code row stride in bytes (D for HND, num_kv_heads * D for NHD); the
// scales of consecutive rows are adjacent for HND and num_kv_heads apart for NHD.
template <int D, bool kNHD, bool kLoadK = true>
__device__ __forceinline__ void load_block_fp8(Fp8Regs<D>& r, const char* kt, const char* vt, const char* kst,
                                               const char* vst, int rows, int q4, int ln, int rs) {
  const int ss = kNHD ? rs / D * 4 : 4;  // scale row stride, bytes
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kt, rows * rs);
  const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vt, rows * rs);
  const __amdgpu_buffer_rsrc_t rks = tile_rsrc(kst, rows * ss);
  const __amdgpu_buffer_rsrc_t rvs = tile_rsrc(vst, rows * ss);
#pragma unroll
  for (int c = 0; c < (kLoadK ? D / 64 : 0); ++c) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, ln * rs + (q4 + 4 * c) * 16, 0, kCacheNT);
    r.k[c] = u32x4{v[0], v[1], v[2], v[3]};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int off = (4 * q4 + i) * rs + ln * (D / 16);
    if constexpr (D / 64 == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, kCacheNT);
      r.v[i][0] = v[0];
      r.v[i][1] = v[1];
    } else {
      r.v[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, kCacheNT);
    }
  }
  if constexpr (kNHD) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.ks[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, (4 * q4 + i) * ss, 0, kCacheNT));
      r.vs[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvs, (4 * q4 + i) * ss, 0, kCacheNT));
    }
  } else {
    const auto ks = __builtin_amdgcn_raw_buffer_load_b128(rks, 16 * q4, 0, kCacheNT);
    const auto vs = __builtin_amdgcn_raw_buffer_load_b128(rvs, 16 * q4, 0, kCacheNT);
    r.ks = f32x4{__uint_as_float(ks[0]), __uint_as_float(ks[1]), __uint_as_float(ks[2]), __uint_as_float(ks[3])};
    r.vs = f32x4{__uint_as_float(vs[0]), __uint_as_float(vs[1]), __uint_as_float(vs[2]), __uint_as_float(vs[3])};
  }
}

// four E4M3 codes (one dword, lowest byte first) -> two dwords of 16-bit
// values, exactly (every E4M3 value is representable in bf16 and fp16)
template <typename T>
__device__ __forceinline__ u32x2 fp8x4_to_16(unsigned w);
template <>
__device__ __forceinline__ u32x2 fp8x4_to_16<__bf16>(unsigned w) {
  return u32x2{__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}
template <>
__device__ __forceinline__ u32x2 fp8x4_to_16<_Float16>(unsigned w) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return u32x2{pack16_exact<_Float16>(lo[0], lo[1]), pack16_exact<_Float16>(hi[0], hi[1])};
}

// four INT8 codes (one dword, lowest byte first, two's complement) -> two
// dwords of 16-bit values, exactly (|code| <= 127 fits bf16 and fp16)
template <typename T>
__device__ __forceinline__ u32x2 int8x4_to_16(unsigned w) {
  const int s = static_cast<int>(w);
  const float f0 = static_cast<float>((s << 24) >> 24), f1 = static_cast<float>((s << 16) >> 24);
  const float f2 = static_cast<float>((s << 8) >> 24), f3 = static_cast<float>(s >> 24);
  return u32x2{pack16_exact<T>(f0, f1), pack16_exact<T>(f2, f3)};
}

// Cache code formats: kQ = 0 (no codes: the cache holds T), kQFp8 (OCP E4M3),
// kQInt8 (signed 8-bit integers). Both code formats keep one fp32 scale per
// token row of one KV head.
constexpr int kQFp8 = 1;
constexpr int kQInt8 = 2;
template <int kQ, typename T>
__device__ __forceinline__ u32x2 codes4_to_16(unsigned w) {
  if constexpr (kQ == kQInt8) return int8x4_to_16<T>(w);
  else return fp8x4_to_16<T>(w);
}

// 8-bit raw block -> the 16-bit operand registers of the MFMA pipeline
template <int kQ, typename T, int D>
__device__ __forceinline__ void codes_to_16(const Fp8Regs<D>& r, BlockRegs<T, D>& o) {
#pragma unroll
  for (int c = 0; c < Shape<T, D>::kNK; ++c) {  // chunk c = code bytes 8c..8c+7 of the lane's slice
    const u32x2 a = codes4_to_16<kQ, T>(r.k[c >> 1][(c & 1) * 2]);
    const u32x2 b = codes4_to_16<kQ, T>(r.k[c >> 1][(c & 1) * 2 + 1]);
    o.k[c] = u32x4{a[0], a[1], b[0], b[1]};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < D / 64; ++w) {
      const u32x2 a = codes4_to_16<kQ, T>(r.v[i][w]);
      o.v[i][2 * w] = a[0];
      o.v[i][2 * w + 1] = a[1];
    }
}

// K chunks of an 8-bit raw block -> the 16-bit A operands of the QK MFMAs
template <int kQ, typename T, int D>
__device__ __forceinline__ void codes_k_to_16(const Fp8Regs<D>& r, BlockRegs<T, D>& o) {
#pragma unroll
  for (int c = 0; c < Shape<T, D>::kNK; ++c) {  // chunk c = code bytes 8c..8c+7 of the lane's slice
    const u32x2 a = codes4_to_16<kQ, T>(r.k[c >> 1][(c & 1) * 2]);
    const u32x2 b = codes4_to_16<kQ, T>(r.k[c >> 1][(c & 1) * 2 + 1]);
    o.k[c] = u32x4{a[0], a[1], b[0], b[1]};
  }
}

// V of a pair of 8-bit raw blocks -> the A operand of each output block mt of
// the 16x16x32 PV MFMA (dwords: rows (0,1) and (2,3) of tile a, then of tile
// b, at element mt). The codes of two rows are interleaved byte by byte
// first, so every converted pair is already (row 2i, row 2i + 1) at one
// element: no 16-bit shuffles after the conversion.
template <int kQ, typename T, int D>
__device__ __forceinline__ void codes_v_operand(const Fp8Regs<D>& a, const Fp8Regs<D>& b, u32x4 (&av)[D / 16]) {
#pragma unroll
  for (int w = 0; w < D / 64; ++w)  // code dword w of a row: elements 4w .. 4w+3
#pragma unroll
    for (int q = 0; q < 4; ++q) {   // dword q of the operand: tile q / 2, rows 2 (q % 2), 2 (q % 2) + 1
      const Fp8Regs<D>& t = q < 2 ? a : b;
      const unsigned c0 = t.v[2 * (q & 1)][w], c1 = t.v[2 * (q & 1) + 1][w];
      const u32x2 lo = codes4_to_16<kQ, T>(__builtin_amdgcn_perm(c1, c0, 0x05010400u));  // elements 4w, 4w+1
      const u32x2 hi = codes4_to_16<kQ, T>(__builtin_amdgcn_perm(c1, c0, 0x07030602u));  // elements 4w+2, 4w+3
      av[4 * w][q] = lo[0];
      av[4 * w + 1][q] = lo[1];
      av[4 * w + 2][q] = hi[0];
      av[4 * w + 3][q] = hi[1];
    }
}

// Quantize values of one token row given the row's absolute maximum and the
// format's largest code Q (448 for E4M3, 127 for INT8): scale = amax / Q,
// inv = Q / amax (both fp32; amax == 0 -> 1, 1), and each code is the nearest
// code to x * inv (ties to even, clamped to +-Q). A row holding a NaN or an
// infinity has no finite scale: it gets scale NaN and every code set to the
// format's marker (E4M3 0x7F, its NaN; INT8 0x80, the one code the rule
// never writes), so every value of the row reads back as NaN. The row
// maximum is taken with an IEEE maximum, which keeps a NaN.
struct RowQuant {
  float scale, inv;
  bool bad;  // the row holds a NaN or an infinity
};
template <int kQ>
constexpr float kQMax = kQ == kQInt8 ? 127.0f : 448.0f;
template <int kQ>
constexpr unsigned kQMarker4 = kQ == kQInt8 ? 0x80808080u : 0x7f7f7f7fu;
template <int kQ>
__device__ __forceinline__ RowQuant row_quant(float amax) {
  if (!(amax <= 3.40282347e38f)) return {__builtin_nanf(""), 1.f, true};
  if (amax == 0.f) return {1.f, 1.f, false};
  return {amax / kQMax<kQ>, kQMax<kQ> / amax, false};
}
template <int kQ>
__device__ __forceinline__ unsigned quant4(float x0, float x1, float x2, float x3, const RowQuant& q) {
  const float inv = q.inv;
  auto c = [inv](float x) { return fminf(fmaxf(x * inv, -kQMax<kQ>), kQMax<kQ>); };
  unsigned r;
  if constexpr (kQ == kQInt8) {
    auto b = [&](float x) { return static_cast<unsigned>(static_cast<int>(__builtin_rintf(c(x)))) & 0xffu; };
    r = b(x0) | (b(x1) << 8) | (b(x2) << 16) | (b(x3) << 24);
  } else {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(c(x0), c(x1), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c(x2), c(x3), w, true);
    r = static_cast<unsigned>(w);
  }
  return q.bad ? kQMarker4<kQ> : r;
}

template <typename T>
__device__ __forceinline__ float elt_to_float(const char* p);
template <>
__device__ __forceinline__ float elt_to_float<float>(const char* p) {
  return *reinterpret_cast<const float*>(p);
}
template <>
__device__ __forceinline__ float elt_to_float<__bf16>(const char* p) {
  return from_bits16<__bf16>(*reinterpret_cast<const unsigned short*>(p));
}
template <>
__device__ __forceinline__ float elt_to_float<_Float16>(const char* p) {
  return from_bits16<_Float16>(*reinterpret_cast<const unsigned short*>(p));
}

template <typename T, int D, bool kCodes>
struct RegsOf {
  using type = BlockRegs<T, D>;
};
template <typename T, int D>
struct RegsOf<T, D, true> {
  using type = Fp8Regs<D>;
};

// ---------------------------------------------------------------------------
// decode partition kernel
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const char* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  char* out;
  float* ws_o;    // [B, Hq, P, D]
  float* ws_lse;  // [B, Hq, P]
  int32_t max_blocks;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;        // Hq / Hkv
  int32_t head_groups;  // ceil(group / 16)
  int32_t num_blocks;
  int32_t pb_per_part;  // 16-row tiles per partition (<= 128)
  int32_t num_parts;    // P
  int32_t tiles_per_block;  // block_size / 16
  int32_t cap_tokens;       // max_blocks * block_size
  float qk_scale;       // scale * log2(e)
  // fused decode step only
  const char* k_new;    // [B, Hkv, D]: newest token's K (written at position n-1)
  const char* v_new;
  char* k_cache_w;      // the caches, writable
  char* v_cache_w;
  int32_t* counters;    // [B, Hkv, head_groups] arrival counters, zero between calls
  int32_t pair_heads;   // 8-bit partition-grouped step: head pairs' workgroups on one XCD
  // FP8 caches only: fp32 scale per (block, KV head, token row)
  const char* k_scales;
  const char* v_scales;
  // chunked prefill only
  const int32_t* q_start;  // [B + 1]: sequence b's query tokens are rows q_start[b] .. q_start[b+1]-1
  int32_t max_q_len;       // bound on q_start[b+1] - q_start[b]
  int32_t q_tiles;         // 16-row query tiles per (sequence, KV head): ceil(max_q_len * group / 16)
};

// Dynamic LDS of the decode kernel when its waves are partitions of one unit
// (fused step): each wave's normalised partial, lane-major per 16-byte chunk,
// then the waves' lse values, then an arrival counter.
extern __shared__ __align__(16) char pkv_dyn_lds[];
// Then the exchange area of a partly filled group's preloaded tile rows
// (128 per wave) and the counter.
constexpr size_t wg_merge_xchg_offset(int waves, int head_dim) {
  return static_cast<size_t>(waves) * (head_dim / 16) * 64 * 16 + static_cast<size_t>(waves) * 16 * 4;
}
constexpr size_t wg_merge_lds_bytes(int waves, int head_dim) {
  return wg_merge_xchg_offset(waves, head_dim) + static_cast<size_t>(waves) * 128 * 4 + 16;
}

// Fused merge of a wave's kR row groups (16 query rows each) over the
// partitions of its work unit `unit`, from the partition kernel itself.
// Partials are stored lane-major per (work unit, row group) (each store
// instruction writes 64 lanes x 16 bytes contiguously) with device-coherent
// stores (sc1: written through the XCD's L2), then the wave drains its stores
// and counts its arrival. The last partition of the unit to arrive reads all
// partials back with device-coherent loads, combines them (exact log-sum-exp
// merge, one online pass over groups of four partitions whose loads are
// issued together), writes the rows through `write_out(rg, 1 / L)` and resets
// the counter for the next call. No L2 write-back or invalidate is needed.
// The workspace comes as plain values (the layout: partials ws_o, lse values
// ws_lse, counters; num_parts slots per unit row group).
struct MergeSpace {
  float* ws_o;
  float* ws_lse;
  int32_t* counters;
  int32_t num_parts;
};
template <int D, int kR, typename WriteOut>
__device__ __forceinline__ void fused_merge(const MergeSpace a, size_t unit, int p, int nparts, int lane,
                                            f32x4 (&acc)[kR][D / 16], const float (&m_run)[kR],
                                            const float (&l_tot)[kR], const float (&inv)[kR], WriteOut& write_out,
                                            const bool (&row_ok)[kR]) {
  constexpr int kE = D / 16;
  constexpr int kChunks = kE;  // 16-byte chunks per lane: 4*E floats
  const int ln = lane & 15;
  const size_t part_stride = static_cast<size_t>(kChunks) * 64 * 16;
  auto rsrc_o = [&](int rg) {
    char* ob = reinterpret_cast<char*>(a.ws_o) + (unit * kR + rg) * a.num_parts * part_stride;
    return tile_rsrc(ob, static_cast<int>(nparts * part_stride));
  };
  auto rsrc_l = [&](int rg) {
    char* lb = reinterpret_cast<char*>(a.ws_lse) + (unit * kR + rg) * a.num_parts * 64;
    return tile_rsrc(lb, nparts * 64);
  };
#pragma unroll
  for (int rg = 0; rg < kR; ++rg) {
    const __amdgpu_buffer_rsrc_t ro = rsrc_o(rg);
    const __amdgpu_buffer_rsrc_t rl = rsrc_l(rg);
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = 4 * k + e;  // value index i * E + mt
        v[e] = acc[rg][idx % kE][idx / kE] * inv[rg];
      }
      if (row_ok[rg])  // a lane holds one query row's values: padding rows are neither stored nor read
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                     __float_as_uint(v[2]), __float_as_uint(v[3])},
                                               ro, (p * kChunks + k) * 1024 + lane * 16, 0, kCacheDeviceCoherent);
    }
    if (lane < 16)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_run[rg] + __builtin_amdgcn_logf(l_tot[rg])), rl,
                                            p * 64 + ln * 4, 0, kCacheDeviceCoherent);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // every store above has completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int32_t* ctr = a.counters + unit;
  int prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __builtin_amdgcn_readfirstlane(prev);  // lane 0 is active here (the unit's first row is real)
  if (prev != nparts - 1) return;
#pragma unroll
  for (int rg = 0; rg < kR; ++rg) {
    const __amdgpu_buffer_rsrc_t ro = rsrc_o(rg);
    const __amdgpu_buffer_rsrc_t rl = rsrc_l(rg);
#pragma unroll
    for (int mt = 0; mt < kE; ++mt) acc[rg][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float M = kNegInf, L = 0.f;
    for (int pp0 = 0; pp0 < nparts; pp0 += 4) {
      float ls[4];
      u32x4 ov[4][kChunks];
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // past the last partition these read as zero
        ls[u] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rl, (pp0 + u) * 64 + ln * 4, 0, kCacheDeviceCoherent));
#pragma unroll
        for (int k = 0; k < kChunks; ++k) {
          u32x4 x = {0u, 0u, 0u, 0u};
          if (row_ok[rg])
            x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              ro, ((pp0 + u) * kChunks + k) * 1024 + lane * 16, 0,
                                              kCacheDeviceCoherent));
          ov[u][k] = x;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) ls[u] = pp0 + u < nparts ? ls[u] : kNegInf;
      const float m_new = fmaxf(M, fmaxf(fmaxf(ls[0], ls[1]), fmaxf(ls[2], ls[3])));
      const float r = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - m_new);
      M = m_new;
      L *= r;
#pragma unroll
      for (int mt = 0; mt < kE; ++mt) acc[rg][mt] *= r;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = __builtin_amdgcn_exp2f(ls[u] - M);  // 0 past the last partition
        L += w;
#pragma unroll
        for (int k = 0; k < kChunks; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int idx = 4 * k + e;
            acc[rg][idx % kE][idx / kE] += w * __uint_as_float(ov[u][k][e]);
          }
      }
    }
    write_out(rg, 1.0f / L);
  }
  if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// What one launch of the tile kernel computes.
enum Mode : int {
  kModeSplit = 0,    // one partition of decode attention; partials go to merge_kernel
  kModeStep = 1,     // fused decode step: append + attention + in-kernel merge
  kModePrefill = 2,  // chunked prefill: causal attention of a chunk's query tokens, in-kernel merge
};

// Row groups (16 query rows each) a prefill wave processes against every
// loaded K/V tile: 4 for 16-bit queries, 2 for fp32 (register budget); one for
// the decode modes.
#ifndef PKV_PREFILL_ROWS
#define PKV_PREFILL_ROWS 4
#endif
template <typename T, int kMode>
constexpr int kPrefillRowGroups = kMode == kModePrefill ? (sizeof(T) == 2 ? PKV_PREFILL_ROWS : 2) : 1;
constexpr int prefill_row_groups(pkv_dtype dtype) { return dtype == PKV_F32 ? 2 : PKV_PREFILL_ROWS; }

// kMode = kModeSplit: one partition of attention (a split sequence leaves
// partials for merge_kernel). kModeStep: the fused decode step -- the partition that
// holds position n-1 also appends the newest token's K/V (written to its slot
// and patched into its registers, never read back), and the last partition of
// a split sequence to finish merges all partitions (arrival counter).
//
// kFp8 = true: the caches hold E4M3 codes with per-row scales (T, the query
// and output type, is bf16 or fp16); each block is converted exactly to T in
// registers, the K scales multiply the scores and the V scales the weights.
//
// kNHD: caches [num_blocks, block_size, Hkv, D] instead of [num_blocks, Hkv,
// block_size, D]. Either way the kernel walks 16-row tiles: a block of
// block_size tokens is block_size / 16 tiles, and a tile is addressed by the
// cache row index (in units of one head's row) of its first token.
//
// kModePrefill: the 16 columns of a wave's score tile are 16 (query token,
// query head) rows of one KV head's group, token-major (row r = token r / g,
// head r % g), and each row sees the keys up to its own position: the chunk's
// query tokens are the last q_len of the sequence's n cached tokens, so token
// i sits at position n - q_len + i and attends to positions 0..n - q_len + i
// (causal attention, "Understanding KV Cache" §1.2; prefill as a matrix
// product over many query positions, "KV Cache and Inference Optimization").
// Decode may run up to PKV_DECODE_WAVES waves per workgroup (the launch's
// blockDim), one per KV head of a group of consecutive heads. For NHD caches,
// whose blocks interleave the heads row by row, the waves together read each
// block's contiguous [rows, heads, D] bytes at about the same time; for HND
// caches they read the adjacent per-head tiles of the same blocks. Four waves
// stay within one wave per SIMD, so the register budget is that of a one-wave
// workgroup. Prefill launches one wave per workgroup.
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4
#endif
#ifndef PKV_WG_PARTS  // HND decode: the waves of a workgroup are partitions of one unit
#define PKV_WG_PARTS 1
#endif
#ifndef PKV_PAIR_HEADS  // 8-bit partition-grouped step: head pairs' workgroups on one XCD
#define PKV_PAIR_HEADS 1
#endif
template <int kMode>
constexpr int kDecodeWaves = kMode == kModePrefill ? 1 : PKV_DECODE_WAVES;

template <typename T, int D, int kMode, int kQ, bool kNHD, bool kWgp = false>
__global__ __launch_bounds__((64 * kDecodeWaves<kMode>)) void decode_partition_kernel(DecodeArgs a) {
  constexpr bool kFp8 = kQ != 0;  // the caches hold 8-bit codes with per-row scales
  constexpr bool kStep = kMode == kModeStep;
  constexpr bool kPrefill = kMode == kModePrefill;
  using S = Shape<T, D>;
  using R = typename RegsOf<T, D, kFp8>::type;
  constexpr bool k16 = sizeof(T) == 2;
  // groups of 16 query rows per wave, all against the same K/V tiles (prefill
  // reuses each loaded tile for kR row groups; decode has one group per wave)
  constexpr int kR = kPrefillRowGroups<T, kMode>;
  static_assert(!kFp8 || k16, "FP8 caches are read with 16-bit queries");
  constexpr int kRowB = kFp8 ? D : S::kRowBytes;  // one head's cached row, bytes
  constexpr int kMaxW = kDecodeWaves<kMode>;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int q4 = lane >> 4;
  const int ln = lane & 15;
  // Partition of this workgroup. Workgroups go to the eight XCDs round-robin
  // by linear id, so with a partition count that is a multiple of 8 partition
  // p of every unit would land on XCD p % 8, and the low partitions, which
  // every sequence has, would crowd the first XCDs. Rotating the partitions
  // by the unit index starts each unit on another XCD.
  //
  // The partition-grouped instance (kWgp: the HND fused step, when the host
  // picks it): the waves are consecutive partitions of one unit (wave w takes
  // partition W * x + w of the workgroup's rotated index x), so a unit's
  // partials meet in the workgroup's LDS instead of global memory. Otherwise
  // (the split path, NHD caches, whose blocks interleave the heads row by
  // row, and grids the host keeps head-grouped): consecutive KV heads of one
  // partition.
  constexpr bool kWgParts = kWgp && kStep && !kNHD && kMaxW > 1;
  const int wv = kMaxW == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int W = static_cast<int>(blockDim.x >> 6);
  const int units_per_head = kPrefill ? a.q_tiles : a.head_groups;  // work units per (sequence, KV head)
  // The workgroup's (partition group, KV head x head group, sequence). 8-bit
  // caches, partition-grouped: the fp32 row scales of KV heads 2i and 2i + 1
  // share each 128-byte line (64 bytes per block and head), and with the
  // heads on different XCDs both L2s fetch the whole line. When the host asks
  // for it (a.pair_heads), the workgroups of such a head pair are renumbered
  // to run back to back on one XCD (linear ids L and L + 8), so the line is
  // fetched once; the pairs still go round-robin over the XCDs.
  int vx = static_cast<int>(blockIdx.x), vy = static_cast<int>(blockIdx.y), vz = static_cast<int>(blockIdx.z);
  if constexpr (kWgParts && kFp8) {
    if (a.pair_heads) {  // the host checked: num_kv_heads even, so gridDim.y is even
      const int gx = static_cast<int>(gridDim.x), gy = static_cast<int>(gridDim.y);
      const int L = vx + gx * (vy + gy * vz);
      const int nwg = gx * gy * static_cast<int>(gridDim.z), main = nwg & ~15;
      int r, mb;  // head pair rank and member
      if (L < main) {
        mb = (L >> 3) & 1;
        r = (L >> 4) * 8 + (L & 7);
      } else {  // the last nwg % 16 workgroups: pairs on consecutive ids
        mb = (L - main) & 1;
        r = (main >> 1) + ((L - main) >> 1);
      }
      const int hp = gy >> 1;  // head pairs x head groups
      vx = r % gx;
      const int rest = r / gx;
      const int yp = rest % hp;
      vz = rest / hp;
      const int pi = yp / units_per_head;
      vy = (2 * pi + mb) * units_per_head + (yp - pi * units_per_head);
    }
  }
  const int xr = PKV_XCD_ROTATE ? (vx + vy + static_cast<int>(gridDim.y) * vz) % static_cast<int>(gridDim.x) : vx;
  const int p = kWgParts ? xr * W + wv : xr;
  const int jg = vy / units_per_head;  // KV head, or group of blockDim / 64 heads
  // head group (decode) or query tile (prefill; in descending order: later
  // tiles see more keys, and the longest workgroups start first)
  const int ui = kPrefill ? units_per_head - 1 - (vy - jg * units_per_head) : vy - jg * units_per_head;
  const int j = (kMaxW == 1 || kWgParts) ? jg : jg * W + wv;
  if constexpr (kWgParts) {  // the LDS arrival counter starts at zero
    if (threadIdx.x == 0) *reinterpret_cast<int*>(pkv_dyn_lds + wg_merge_lds_bytes(W, D) - 16) = 0;
    __syncthreads();
  }
  const int hg = kPrefill ? 0 : ui;
  const int b = vz;

  const int cap = a.cap_tokens;
  int blk0 = p * a.pb_per_part;  // first tile of the partition
  const int row_step = kNHD ? a.num_kv_heads : 1;  // cache rows between consecutive tokens of one head
  // First cache row of each of this partition's tiles (lane i: tile blk0 + i,
  // and blk0 + 64 + i for partitions longer than 64 tiles), -1 where the
  // table names a block outside the pool. The sequence length (a scalar
  // load) and the table entries are requested together, bounded by the table
  // width rather than by the length, and nothing is computed on an entry
  // inside a lane-dependent branch, so the first K/V loads wait for one round
  // trip, not two.
  // (a vector-memory load, so that it is issued beside the table loads and
  // shares their wait; as a scalar load it was placed after that wait)
  int n = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(
      tile_rsrc(reinterpret_cast<const char*>(a.context_lens), (b + 1) * 4), b * 4, 0, 0));
  const size_t trow = static_cast<size_t>(b) * a.max_blocks;
  const int m = a.tiles_per_block;
  const int max_tiles = a.max_blocks * m;
  auto table_id = [&](int lt) -> int {  // every lane loads (an in-range entry); out-of-range tiles get -1
    const int lbc = min(lt, max_tiles - 1) / m;
    const int id = a.block_tables[trow + lbc];
    return lt < max_tiles ? id : -1;
  };
  auto row_of = [&](int id, int lt) -> int {
    if (static_cast<unsigned>(id) >= static_cast<unsigned>(a.num_blocks)) return -1;
    const int sub = lt - (lt / m) * m;
    return kNHD ? (id * m + sub) * kTile * a.num_kv_heads + j : ((id * a.num_kv_heads + j) * m + sub) * kTile;
  };
  const int raw0 = table_id(blk0 + lane);  // an unconditional load: its wait falls at the first use
  const int id0 = lane < a.pb_per_part ? raw0 : -1;
  int id1 = -1;
  if (a.pb_per_part > 64) {  // wave-uniform
    const int raw1 = table_id(blk0 + 64 + lane);
    id1 = 64 + lane < a.pb_per_part ? raw1 : -1;
  }
  __builtin_amdgcn_sched_barrier(0);  // the length and table loads are issued before any wait on them
  n = __builtin_amdgcn_readfirstlane(n);
  int my_r0 = row_of(id0, blk0 + lane), my_r02 = row_of(id1, blk0 + 64 + lane);
  // a length past the table's capacity is clamped for reading; the fused
  // step then appends nothing (position n - 1 is not the new token's)
  const bool len_fits = n <= cap;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  // prefill: this wave's 16 * kR query rows, their key limits, and the wave's span
  int q_tok0 = 0, min_limit = 0;
  int my_limit[kR], row_tok[kR], row_hin[kR];
  bool row_ok[kR];
#pragma unroll
  for (int rg = 0; rg < kR; ++rg) {
    my_limit[rg] = 0;
    row_tok[rg] = 0;
    row_hin[rg] = 0;
    row_ok[rg] = true;
  }
  if constexpr (kPrefill) {
    q_tok0 = a.q_start[b];
    int q_len = a.q_start[b + 1] - q_tok0;
    q_len = q_len < 0 ? 0 : min(q_len, min(a.max_q_len, n));
    const int rows = q_len * a.group;
    const int r0 = ui * kTile * kR;  // the wave's first row
    const int first = n - q_len;     // position of the chunk's first token
#pragma unroll
    for (int rg = 0; rg < kR; ++rg) {
      const int r = r0 + rg * kTile + ln;
      row_ok[rg] = r < rows;
      row_tok[rg] = r / a.group;
      row_hin[rg] = r - row_tok[rg] * a.group;
      my_limit[rg] = row_ok[rg] ? first + row_tok[rg] + 1 : 0;
    }
    min_limit = first + r0 / a.group + 1;
    // the wave reads keys up to its last row's position (none if it has no rows)
    n = r0 < rows ? first + min(r0 + kTile * kR - 1, rows - 1) / a.group + 1 : 0;
    if (n == 0) return;  // no rows: the unit does nothing (its merge counter stays untouched)
  }
  const int nblk_seq = (n + kTile - 1) / kTile;  // tiles the wave reads
  int nparts = nblk_seq == 0 ? 1 : (nblk_seq + a.pb_per_part - 1) / a.pb_per_part;
  int nblk = 0;
  int ngroups = 1;  // partition-grouped workgroups of a unit (fused step)
  bool grouped = false;
  if constexpr (kWgParts) {  // wave-uniform
    // The unit's tiles in groups of W full partitions, one group per
    // workgroup. A group that the sequence fills only in part (its last,
    // or a short sequence's only group) splits its tiles evenly over all W
    // waves; the waves exchange their preloaded tile rows through LDS, so
    // no wave waits for a second table read and no wave sits idle.
    const int gt = W * a.pb_per_part;  // tiles of a full group
    if (nblk_seq == 0) {  // nothing to read: one wave writes the zero row
      if (wv != 0) return;
      nparts = 1;
    } else {
      grouped = true;
      ngroups = (nblk_seq + gt - 1) / gt;
      if (xr >= ngroups) return;  // the whole workgroup
      nparts = W * ngroups;
      const int g0 = xr * gt;
      const int len = min(gt, nblk_seq - g0);
      if (len < gt) {  // workgroup-uniform
        const int base = len / W, rem = len % W;
        blk0 = g0 + wv * base + min(wv, rem);
        nblk = base + (wv < rem ? 1 : 0);
        int* xt = reinterpret_cast<int*>(pkv_dyn_lds + wg_merge_xchg_offset(W, D));  // [W][pb_per_part]
        if (lane < a.pb_per_part) xt[wv * a.pb_per_part + lane] = my_r0;
        if (64 + lane < a.pb_per_part) xt[wv * a.pb_per_part + 64 + lane] = my_r02;
        __syncthreads();
        const int off = blk0 - g0;
        my_r0 = lane < nblk ? xt[off + lane] : -1;
        my_r02 = 64 + lane < nblk ? xt[off + 64 + lane] : -1;
      } else {
        nblk = a.pb_per_part;
      }
    }
  }
  if (!grouped) {
    if (p >= nparts) return;
    nblk = min(a.pb_per_part, nblk_seq - blk0);  // may be 0 only when n == 0
  }
  auto tile_r0 = [&](int t) -> int {  // t wave-uniform, < 128
    return t < 64 ? __builtin_amdgcn_readlane(my_r0, t & 63) : __builtin_amdgcn_readlane(my_r02, t & 63);
  };

  // Fused append: the partition holding position n-1 takes the new token's
  // K/V from k_new/v_new and uses them from registers. They are read here,
  // right after the table (so no earlier wait covers them); 8-bit rows are
  // quantized once the first tile loads are out, and the row is written to
  // its slot after the loop, where the store's completion overlaps the
  // merge's own wait.
  const bool has_new = kStep && n > 0 && len_fits && nblk > 0 && blk0 + nblk == nblk_seq;
  const int new_t = has_new ? (n - 1) / kTile - blk0 : -1;  // tile index inside the partition
  const int new_row = (n - 1) % kTile;
  u32x4 kn[S::kNK];   // 16-bit caches: the new K in the tile's chunk order
  unsigned vn[S::kVDW];
  constexpr int kNewK = kFp8 ? D / 32 : 1;  // 8-bit caches: this lane's D/4 16-bit K values (its K chunks)
  u32x4 knr[kNewK];
  unsigned vnr[kFp8 ? D / 32 : 1];          // and its D/16 V values
  u32x4 kn8[D / 64];  // 8-bit: the quantized K chunks and V codes of the new row
  unsigned vn8[D / 64];
  float ks_new = 1.f, vs_new = 1.f;
  if constexpr (kStep) {
    if (has_new) {  // wave-uniform
      const size_t src = (static_cast<size_t>(b) * a.num_kv_heads + j) * S::kRowBytes;
      if constexpr (kFp8) {
#pragma unroll
        for (int c = 0; c < kNewK; ++c)
          knr[c] = *reinterpret_cast<const u32x4*>(a.k_new + src + k_slice_elt<D>(q4, 8 * c) * S::kElt);
        const char* vsrc = a.v_new + src + ln * (D / 16) * S::kElt;
        if constexpr (D / 32 == 4) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(vsrc);
          vnr[0] = x[0];
          vnr[1] = x[1];
          vnr[2] = x[2];
          vnr[3] = x[3];
        } else {
          const u32x2 x = *reinterpret_cast<const u32x2*>(vsrc);
          vnr[0] = x[0];
          vnr[1] = x[1];
        }
      } else {
#pragma unroll
        for (int c = 0; c < S::kNK; ++c) kn[c] = *reinterpret_cast<const u32x4*>(a.k_new + src + (4 * c + q4) * 16);
        const char* vsrc = a.v_new + src + ln * S::kE * S::kElt;
        if constexpr (S::kVDW == 2) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(vsrc);
          vn[0] = w[0];
          vn[1] = w[1];
        } else {
#pragma unroll
          for (int w = 0; w < S::kVDW; w += 4) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(vsrc + w * 4);
            vn[w] = x[0];
            vn[w + 1] = x[1];
            vn[w + 2] = x[2];
            vn[w + 3] = x[3];
          }
        }
      }
    }
  }
  // 8-bit caches: quantize the new K and V rows (scale = row amax / Q)
  auto quantize_new = [&]() __attribute__((always_inline)) {
    if constexpr (kStep && kFp8) {
      // K: this lane's D/4 values (its K chunks); the row maximum spans the 4 quarters
      float kx[D / 4];
#pragma unroll
      for (int c = 0; c < kNewK; ++c)
#pragma unroll
        for (int h = 0; h < 8; ++h) kx[8 * c + h] = from_bits16<T>((knr[c][h >> 1] >> (16 * (h & 1))) & 0xffffu);
      float am = 0.f;
#pragma unroll
      for (int e = 0; e < D / 4; ++e) am = fmax_nan(am, fabsf(kx[e]));
      am = fmax_nan(am, xor_shuffle(am, 16));
      am = fmax_nan(am, xor_shuffle(am, 32));
      const RowQuant kq = row_quant<kQ>(am);
      ks_new = kq.scale;
#pragma unroll
      for (int c = 0; c < D / 64; ++c) {
        unsigned w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
          w[d] = quant4<kQ>(kx[16 * c + 4 * d], kx[16 * c + 4 * d + 1], kx[16 * c + 4 * d + 2], kx[16 * c + 4 * d + 3],
                            kq);
        kn8[c] = u32x4{w[0], w[1], w[2], w[3]};
      }
      // V: this lane's D/16 values [ln*D/16, ...); the maximum spans the 16 lanes of a quarter
      float vx[D / 16];
#pragma unroll
      for (int e = 0; e < D / 16; ++e) vx[e] = from_bits16<T>((vnr[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      float vm = 0.f;
#pragma unroll
      for (int e = 0; e < D / 16; ++e) vm = fmax_nan(vm, fabsf(vx[e]));
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) vm = fmax_nan(vm, xor_shuffle(vm, m));
      const RowQuant vq = row_quant<kQ>(vm);
      vs_new = vq.scale;
#pragma unroll
      for (int w = 0; w < D / 64; ++w)
        vn8[w] = quant4<kQ>(vx[4 * w], vx[4 * w + 1], vx[4 * w + 2], vx[4 * w + 3], vq);
    }
  };

  // this lane's query row (column of the score tile): a head of the GQA group
  // (decode) or a (token, head) pair of the chunk (prefill); qidx indexes the
  // [*, Hq] rows of q and out
  bool head_ok[kR];
  size_t qidx[kR];
  u32x4 qv[kR][S::kNK];  // Q as the B operand, same chunk permutation as K
#pragma unroll
  for (int rg = 0; rg < kR; ++rg) {
    const int hin = kPrefill ? row_hin[rg] : hg * 16 + ln;  // head index inside the GQA group
    head_ok[rg] = kPrefill ? row_ok[rg] : hin < a.group;
    const int hq = j * a.group + (head_ok[rg] ? hin : 0);
    qidx[rg] = kPrefill ? (static_cast<size_t>(q_tok0) + (head_ok[rg] ? row_tok[rg] : 0)) * a.num_heads + hq
                        : static_cast<size_t>(b) * a.num_heads + hq;
    const char* qrow = a.q + qidx[rg] * S::kRowBytes;
#pragma unroll
    for (int c = 0; c < S::kNK; ++c) {
      // byte offset of 16-byte chunk c: same-type caches (4c + q4) * 16 (the K
      // tile's chunk order); 8-bit caches (T is 16-bit) the 8 elements of MFMA
      // chunk c of the lane's K codes
      const int off = kFp8 ? k_slice_elt<D>(q4, 8 * c) * 2 : (4 * c + q4) * 16;
      qv[rg][c] = head_ok[rg] ? *reinterpret_cast<const u32x4*>(qrow + off) : u32x4{0, 0, 0, 0};
    }
  }

  f32x4 acc[kR][S::kE];
  float m_run[kR];  // running max of scaled scores (log2 units)
  float l_run[kR];  // this lane's share of the running denominator
#pragma unroll
  for (int rg = 0; rg < kR; ++rg) {
#pragma unroll
    for (int mt = 0; mt < S::kE; ++mt) acc[rg][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rg] = kNegInf;
    l_run[rg] = 0.f;
  }

  // First cache row of the partition's tile t and how many of its token rows
  // to fetch: 0 past the partition end or for an out-of-range id (nothing is
  // read then), else the tile's tokens below n.
  const int rs = kRowB * row_step;  // bytes between consecutive token rows of one head
  auto block_src = [&](int t, int& rows) -> size_t {
    const int r0 = tile_r0(min(t, 127));
    const bool ok = t < nblk && r0 >= 0;
    rows = ok ? min(kTile, n - (blk0 + t) * kTile) : 0;
    if (kStep && t == new_t) rows = new_row;  // the new row comes from registers
    return ok ? static_cast<size_t>(r0) : 0;
  };
  // 8-bit K of head size 128 in HND caches goes through a per-wave LDS ring
  // (one 2 KiB slot per ring tile, in the dynamic LDS after the workgroup
  // merge area). Read straight into registers, a lane's K takes 64 bytes of
  // each of 16 rows per load, which measured 4-5% of the stream rate below
  // 1 KiB-contiguous loads; here every load takes 8 whole rows and the MFMA
  // operands come back with one LDS read per 16-byte chunk. Slot byte
  // 1024 h + 16 (8 r + (c ^ r)) holds chunk c of tile row 8 h + r (r < 8), so
  // the reads of 8 consecutive lanes (rows r = 0..7, one chunk each) fall in 8
  // different 16-byte bank groups.
  constexpr bool kKLds = kFp8 && !kNHD && D == 128 && !kPrefill && PKV_KRING_8BIT && PKV_DECODE_PAIRS;
  char* const kring = pkv_dyn_lds + (kWgParts ? wg_merge_lds_bytes(W, D) : 0) + wv * kKRingWaveBytes;
  auto load_ring = [&](int slot, R& r, size_t row0, int rows) {
    if constexpr (kKLds) {
      const __amdgpu_buffer_rsrc_t rk = tile_rsrc(a.k_cache + row0 * D, rows * rs);
      char* const kl = kring + slot * (16 * D);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * h + (lane >> 3), chunk = (lane & 7) ^ (lane >> 3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, lds_ptr(kl + h * 1024), 16, row * rs + chunk * 16, 0, 0,
                                                 kCacheNT);
      }
      // the tile's V and scale loads (kRingVSLoads of them) are issued after
      // its K loads: read_k's wait counts on that order
      __builtin_amdgcn_sched_barrier(0);
      load_block_fp8<D, kNHD, false>(r, a.k_cache + row0 * D, a.v_cache + row0 * D, a.k_scales + row0 * 4,
                                     a.v_scales + row0 * 4, rows, q4, ln, rs);
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (kFp8) {
      (void)slot;
      load_block_fp8<D, kNHD>(r, a.k_cache + row0 * D, a.v_cache + row0 * D, a.k_scales + row0 * 4,
                              a.v_scales + row0 * 4, rows, q4, ln, rs);
    } else {
      (void)slot;
      load_block<T, D>(r, a.k_cache + row0 * S::kRowBytes, a.v_cache + row0 * S::kRowBytes, rows, q4, ln, rs);
    }
  };
  // Loads into LDS are not waited for by the compiler, so before a pair's K
  // is read the wave drains its own loads down to those issued after that
  // pair's last K load: the last tile's V and scale loads, then the next
  // pair's loads (issued first, so that two pairs stay in flight)
  constexpr int kRingVSLoads = 4 + 2;  // V: four 8-byte row loads; scales: two 16-byte loads (HND)
  constexpr int kRingNewer = kRingVSLoads + 2 * (2 + kRingVSLoads);
  static_assert(kRingNewer < 64, "vmcnt field");
  auto wait_ring_k = [&]() __attribute__((always_inline)) {
    if constexpr (kKLds) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      // vmcnt <= kRingNewer (bits 3:0 and 15:14), expcnt and lgkmcnt: no wait
      __builtin_amdgcn_s_waitcnt(((kRingNewer & 0x30) << 10) | 0xF70 | (kRingNewer & 0xF));
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
  };
  // the ring slot's K into the MFMA operand registers: lane (q4, r) takes
  // chunks q4 and q4 + 4 of tile row r
  auto read_k = [&](int slot, R& r) __attribute__((always_inline)) {
    if constexpr (kKLds) {
      const char* const kl = kring + slot * (16 * D) + (ln >> 3) * 1024 + (ln & 7) * 128;
#pragma unroll
      for (int c = 0; c < 2; ++c) r.k[c] = *reinterpret_cast<const u32x4*>(kl + 16 * ((q4 + 4 * c) ^ (ln & 7)));
    } else {
      (void)slot;
      (void)r;
    }
  };

  // fused step: the tile holding position n-1 gets the appended token's row
  // from registers (it was not fetched)
  auto patch_new = [&](R& rr, int& valid, int t) {
    if constexpr (kStep) {
      if (t == new_t) {  // wave-uniform
        valid = new_row + 1;
        if constexpr (kFp8) {
          if (ln == new_row) {
#pragma unroll
            for (int c = 0; c < D / 64; ++c) rr.k[c] = kn8[c];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * q4 + i == new_row) {
#pragma unroll
              for (int w = 0; w < D / 64; ++w) rr.v[i][w] = vn8[w];
              rr.ks[i] = ks_new;
              rr.vs[i] = vs_new;
            }
        } else {
          if (ln == new_row) {
#pragma unroll
            for (int c = 0; c < S::kNK; ++c) rr.k[c] = kn[c];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * q4 + i == new_row) {
#pragma unroll
              for (int w = 0; w < S::kVDW; ++w) rr.v[i][w] = vn[w];
            }
        }
      }
    }
  };
  auto process = [&](R& rr, int valid, int t) {  // valid: token rows of this block in range
    patch_new(rr, valid, t);
    BlockRegs<T, D> conv;
    BlockRegs<T, D>* rp;
    if constexpr (kFp8) {
      codes_to_16<kQ, T, D>(rr, conv);
      rp = &conv;
    } else {
      rp = &rr;
    }
    BlockRegs<T, D>& r = *rp;
#pragma unroll
    for (int rg = 0; rg < kR; ++rg) {
    // scores
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (k16) {
#pragma unroll
      for (int c = 0; c < S::kNK; ++c) s = mfma_qk16<T>(r.k[c], qv[rg][c], s);
    } else {
#pragma unroll
      for (int c = 0; c < S::kNK; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(r.k[c][e]), __uint_as_float(qv[rg][c][e]), s, 0, 0,
                                                   0);
    }
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kFp8) sc[i] = s[i] * rr.ks[i] * a.qk_scale;
      else sc[i] = s[i] * a.qk_scale;
    }
    if (valid < kTile) {  // wave-uniform: the last tile of a sequence, or a bad id
      // rows past `valid` were not fetched (K and V read as zero), so no NaN
      // padding enters the MFMAs; their scores are selected out here
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = 4 * q4 + i < valid ? sc[i] : kNegInf;
    }
    if constexpr (kPrefill) {
      const int key0 = (blk0 + t) * kTile;
      if (key0 + kTile > min_limit) {  // wave-uniform: some row's causal limit falls inside this tile
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = key0 + 4 * q4 + i < my_limit[rg] ? sc[i] : kNegInf;
      }
    }
    const float mx = row_max4(fmax_nan(fmax_nan(sc[0], sc[1]), fmax_nan(sc[2], sc[3])));
    // Lazy rescaling: the reference maximum m_run only moves when a head's
    // block maximum exceeds it by more than kRescaleSlack (log2 units), so the
    // weights stay <= 2^kRescaleSlack and the accumulator is rescaled rarely.
    // Any reference gives the same softmax; this one keeps exp2 in range.
    const bool grow = mx > m_run[rg] + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform
      const float m_new = grow ? mx : m_run[rg];
      const float alpha = m_run[rg] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run[rg] - m_new);
#pragma unroll
      for (int mt = 0; mt < S::kE; ++mt) acc[rg][mt] *= alpha;
      l_run[rg] *= alpha;
      m_run[rg] = m_new;
    }
    const float m_use = m_run[rg] == kNegInf ? 0.f : m_run[rg];
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(sc[i] - m_use);
    if constexpr (k16) {
      // P^T operand: each weight is split into a 16-bit head plus a 16-bit
      // residual (two MFMAs against the same V tile), so the weights carry
      // about 16 significant bits instead of 8 (bf16) or 11 (fp16)
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = pr[i];
        if constexpr (kFp8) pv[i] *= rr.vs[i];  // FP8: the V scale rides on the weight
      }
      l_run[rg] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      unsigned hi[2], lo[2];
      split16_pair<T>(pv[0], pv[1], hi[0], lo[0]);
      split16_pair<T>(pv[2], pv[3], hi[1], lo[1]);
      const u32x2 pw_hi = {hi[0], hi[1]};
      const u32x2 pw_lo = {lo[0], lo[1]};
#pragma unroll
      for (int mt = 0; mt < S::kE; ++mt) {
        const unsigned sel = (mt & 1) ? 0x07060302u : 0x05040100u;
        const u32x2 av = {__builtin_amdgcn_perm(r.v[1][mt >> 1], r.v[0][mt >> 1], sel),
                          __builtin_amdgcn_perm(r.v[3][mt >> 1], r.v[2][mt >> 1], sel)};
        acc[rg][mt] = mfma_pv16<T>(av, pw_hi, acc[rg][mt]);
        acc[rg][mt] = mfma_pv16<T>(av, pw_lo, acc[rg][mt]);
      }
    } else {
      l_run[rg] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < S::kE; ++mt)
          acc[rg][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(r.v[i][mt]), pr[i], acc[rg][mt], 0, 0, 0);
    }
    }  // row groups
  };

  // With 16-bit queries tiles are taken in pairs: one softmax step (one
  // cross-lane maximum, one rescale decision) per 32 keys, and one 16x16x32
  // PV MFMA per output block over both tiles. The MFMA's K index runs over
  // tile a's rows 4*q4 .. 4*q4+3, then tile b's: each lane already holds those
  // V rows and those weights, so neither operand moves between lanes.
  constexpr bool kPairs = k16 && (kPrefill ? PKV_PREFILL_PAIRS : PKV_DECODE_PAIRS);
  auto process_pair = [&](R& ra, int va, int ta, R& rb, int vb, int tb) {
    if constexpr (kPairs) {  // (16-bit queries only: the fp32 build must not instantiate it)
      patch_new(ra, va, ta);
      patch_new(rb, vb, tb);
      BlockRegs<T, D> ca, cb;
      BlockRegs<T, D>* pa;
      BlockRegs<T, D>* pb2;
      // V operands over both tiles, shared by the row groups
      u32x4 av[S::kE];
      if constexpr (kFp8) {
        codes_k_to_16<kQ, T, D>(ra, ca);
        codes_k_to_16<kQ, T, D>(rb, cb);
        codes_v_operand<kQ, T, D>(ra, rb, av);
        pa = &ca;
        pb2 = &cb;
      } else {
        pa = &ra;
        pb2 = &rb;
#pragma unroll
        for (int mt = 0; mt < S::kE; ++mt) {
          const unsigned sel = (mt & 1) ? 0x07060302u : 0x05040100u;
          av[mt] = u32x4{__builtin_amdgcn_perm(ra.v[1][mt >> 1], ra.v[0][mt >> 1], sel),
                         __builtin_amdgcn_perm(ra.v[3][mt >> 1], ra.v[2][mt >> 1], sel),
                         __builtin_amdgcn_perm(rb.v[1][mt >> 1], rb.v[0][mt >> 1], sel),
                         __builtin_amdgcn_perm(rb.v[3][mt >> 1], rb.v[2][mt >> 1], sel)};
        }
      }
      BlockRegs<T, D>& A = *pa;
      BlockRegs<T, D>& Bt = *pb2;
      const int key_a = (blk0 + ta) * kTile, key_b = (blk0 + tb) * kTile;
#pragma unroll
      for (int rg = 0; rg < kR; ++rg) {
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < S::kNK; ++c) {
          sa = mfma_qk16<T>(A.k[c], qv[rg][c], sa);
          sb = mfma_qk16<T>(Bt.k[c], qv[rg][c], sb);
        }
        float sc[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (kFp8) {
            sc[i] = sa[i] * ra.ks[i] * a.qk_scale;
            sc[4 + i] = sb[i] * rb.ks[i] * a.qk_scale;
          } else {
            sc[i] = sa[i] * a.qk_scale;
            sc[4 + i] = sb[i] * a.qk_scale;
          }
        }
        // rows past a tile's valid count were not fetched; keys past a row's
        // position are masked (both tests are wave-uniform to enter)
        if (va < kTile || (kPrefill && key_a + kTile > min_limit)) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[i] = (4 * q4 + i < va && (!kPrefill || key_a + 4 * q4 + i < my_limit[rg])) ? sc[i] : kNegInf;
        }
        if (vb < kTile || (kPrefill && key_b + kTile > min_limit)) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sc[4 + i] = (4 * q4 + i < vb && (!kPrefill || key_b + 4 * q4 + i < my_limit[rg])) ? sc[4 + i] : kNegInf;
        }
        const float mx = row_max4(fmax_nan(fmax_nan(fmax_nan(sc[0], sc[1]), fmax_nan(sc[2], sc[3])),
                                           fmax_nan(fmax_nan(sc[4], sc[5]), fmax_nan(sc[6], sc[7]))));
        const bool grow = mx > m_run[rg] + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform
          const float m_new = grow ? mx : m_run[rg];
          const float alpha = m_run[rg] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run[rg] - m_new);
#pragma unroll
          for (int mt = 0; mt < S::kE; ++mt) acc[rg][mt] *= alpha;
          l_run[rg] *= alpha;
          m_run[rg] = m_new;
        }
        const float m_use = m_run[rg] == kNegInf ? 0.f : m_run[rg];
        float pv[8];
        float lsum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pr = __builtin_amdgcn_exp2f(sc[i] - m_use);
          lsum += pr;
          pv[i] = pr;
          if constexpr (kFp8) pv[i] *= i < 4 ? ra.vs[i] : rb.vs[i - 4];
        }
        l_run[rg] += lsum;
        unsigned hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split16_pair<T>(pv[2 * i], pv[2 * i + 1], hi[i], lo[i]);
        const u32x4 pw_hi = {hi[0], hi[1], hi[2], hi[3]}, pw_lo = {lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
        for (int mt = 0; mt < S::kE; ++mt) {
          acc[rg][mt] = mfma_qk16<T>(av[mt], pw_hi, acc[rg][mt]);
          acc[rg][mt] = mfma_qk16<T>(av[mt], pw_lo, acc[rg][mt]);
        }
      }
    }
  };

  // Stream the partition's blocks through a register ring that keeps kAhead
  // blocks of K/V loads in flight while the oldest block is consumed. Loads
  // are issued unconditionally (past the partition end they fetch nothing, see
  // load_block) so that every iteration issues the same loads and the compiler
  // can wait on a precise outstanding-load count.
  constexpr int kAhead = kPrefill ? (sizeof(T) == 2 ? PKV_AHEAD_PREFILL : PKV_AHEAD_32BIT)
                                  : (kFp8 ? PKV_AHEAD_FP8 : (sizeof(T) == 2 ? PKV_AHEAD_16BIT : PKV_AHEAD_32BIT));
  constexpr int kRing = kAhead + 1;
  // pairs held by the ring: kNP - 1 pairs in flight while one is consumed
  constexpr int kNP = kFp8 ? PKV_PAIR_RING_8BIT : PKV_PAIR_RING;
  R ring[kPairs ? 2 * kNP : kRing];
  int ring_rows[kPairs ? 2 * kNP : kRing];
  if constexpr (kPairs) {
    if (nblk > 0) {
#pragma unroll
      for (int u = 0; u < 2 * (kNP - 1); ++u) {
        const size_t tile = block_src(u, ring_rows[u]);
        load_ring(u, ring[u], tile, ring_rows[u]);
      }
      // 8-bit caches: the new row, read right after the table, is quantized
      // while the first tiles are in flight (only the quantized row stays live)
      __builtin_amdgcn_sched_barrier(0);
      if (has_new) quantize_new();
      for (int t0 = 0; t0 < nblk; t0 += 2 * kNP) {
#pragma unroll
        for (int pp = 0; pp < kNP; ++pp) {
          const int cur = 2 * pp, nxt = 2 * ((pp + kNP - 1) % kNP);  // slot of the pair kNP - 1 ahead
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const size_t tile = block_src(t0 + 2 * (pp + kNP - 1) + u, ring_rows[nxt + u]);
            load_ring(nxt + u, ring[nxt + u], tile, ring_rows[nxt + u]);
          }
          __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before any wait below
          if (t0 + 2 * pp < nblk) {  // wave-uniform
            // the LDS-ring K of this pair (its slots were last read a pair ago)
            wait_ring_k();
            read_k(cur, ring[cur]);
            read_k(cur + 1, ring[cur + 1]);
            process_pair(ring[cur], ring_rows[cur], t0 + 2 * pp, ring[cur + 1], ring_rows[cur + 1], t0 + 2 * pp + 1);
          }
        }
      }
      if constexpr (kKLds) __builtin_amdgcn_s_waitcnt(0xF70);  // no load into LDS outlives the loop
    }
  } else if (nblk > 0) {  // wave-uniform; nblk == 0 only for an empty sequence
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const size_t tile = block_src(u, ring_rows[u]);
      load_ring(u, ring[u], tile, ring_rows[u]);
    }
    // several ring rotations per loop iteration: only the first block after
    // the back-edge may see a conservative wait
    constexpr int kUnroll = kRing * PKV_RING_ROTATIONS;
    for (int t0 = 0; t0 < nblk; t0 += kUnroll) {
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu) {
        const int u = uu % kRing;
        const int slot = (u + kAhead) % kRing;
        const size_t tile = block_src(t0 + uu + kAhead, ring_rows[slot]);
        load_ring(slot, ring[slot], tile, ring_rows[slot]);
        __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before any wait below
        if (t0 + uu < nblk) process(ring[u], ring_rows[u], t0 + uu);
      }
    }
  }

  // fused append: the new K/V (codes and scales for 8-bit caches) into the
  // slot of position n-1 (head group 0 writes; the others only read)
  if constexpr (kStep) {
    const int r0 = has_new ? tile_r0(new_t) : -1;
    if (has_new && hg == 0 && r0 >= 0) {  // wave-uniform
      const size_t row = static_cast<size_t>(r0) + static_cast<size_t>(new_row) * row_step;
      if constexpr (kFp8) {
        if (ln == 0) {
#pragma unroll
          for (int c = 0; c < D / 64; ++c)
            *reinterpret_cast<u32x4*>(a.k_cache_w + row * D + (q4 + 4 * c) * 16) = kn8[c];
        }
        if (q4 == 0) {
          char* vd = a.v_cache_w + row * D + ln * (D / 16);
          if constexpr (D / 64 == 2) *reinterpret_cast<u32x2*>(vd) = u32x2{vn8[0], vn8[1]};
          else *reinterpret_cast<unsigned*>(vd) = vn8[0];
        }
        if (lane == 0) {
          reinterpret_cast<float*>(const_cast<char*>(a.k_scales))[row] = ks_new;
          reinterpret_cast<float*>(const_cast<char*>(a.v_scales))[row] = vs_new;
        }
      } else {
        const size_t dst = row * S::kRowBytes;
        if (ln == 0) {
#pragma unroll
          for (int c = 0; c < S::kNK; ++c) *reinterpret_cast<u32x4*>(a.k_cache_w + dst + (4 * c + q4) * 16) = kn[c];
        }
        if (q4 == 0) store_dwords<S::kVDW>(a.v_cache_w + dst + ln * S::kE * S::kElt, vn);
      }
    }
  }

  // combine the four lanes' partial denominators of each row
  float l_tot[kR], inv[kR];
#pragma unroll
  for (int rg = 0; rg < kR; ++rg) {
    l_tot[rg] = l_run[rg] + xor_shuffle(l_run[rg], 16);
    l_tot[rg] += xor_shuffle(l_tot[rg], 32);
    inv[rg] = l_tot[rg] > 0.f ? 1.0f / l_tot[rg] : 0.f;
  }
  if constexpr (kR == 1) {
    if (!head_ok[0]) return;  // padding heads of the group: nothing to store
  }

  // this lane's 4 x E output values of row group rg (d = (4*q4 + i) * E + mt), scaled, to `out`
  auto write_out = [&](int rg, float scale_by) {
    if (!head_ok[rg]) return;
    char* orow = a.out + qidx[rg] * S::kRowBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = (4 * q4 + i) * S::kE;
      unsigned w[S::kVDW];
      if constexpr (k16) {
#pragma unroll
        for (int mt = 0; mt < S::kE; mt += 2)
          w[mt >> 1] =
              to_bits16<T>(acc[rg][mt][i] * scale_by) | (to_bits16<T>(acc[rg][mt + 1][i] * scale_by) << 16);
      } else {
#pragma unroll
        for (int mt = 0; mt < S::kE; ++mt) w[mt] = __float_as_uint(acc[rg][mt][i] * scale_by);
      }
      store_dwords<S::kVDW>(orow + d0 * S::kElt, w);
    }
  };

  if (nparts == 1) {
#pragma unroll
    for (int rg = 0; rg < kR; ++rg) write_out(rg, inv[rg]);
    return;
  }
  if constexpr (kWgParts) {
    if (grouped) {  // wave-uniform
      // Merge the workgroup's partitions of this unit in LDS: each wave leaves
      // its normalised partial and lse, counts its arrival, and the last of the
      // `active` waves combines them (exact log-sum-exp merge). A unit whose
      // partitions span several workgroups then merges the workgroup results
      // through global memory (fused_merge), one partial per workgroup.
      const int active = W;  // every wave of the group takes part (some with no tiles: lse = -inf)
      const size_t unit = (static_cast<size_t>(b) * a.num_kv_heads + j) * units_per_head + ui;
      const MergeSpace ms{a.ws_o, a.ws_lse, a.counters, a.num_parts};
      if (active > 1) {
        constexpr int kE = S::kE;
        f32x4* po = reinterpret_cast<f32x4*>(pkv_dyn_lds);                       // [W][kE][64]
        float* pl = reinterpret_cast<float*>(pkv_dyn_lds + static_cast<size_t>(W) * kE * 64 * 16);  // [W][16]
        int* ctr = reinterpret_cast<int*>(pkv_dyn_lds + wg_merge_lds_bytes(W, D) - 16);
#pragma unroll
        for (int k = 0; k < kE; ++k) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int idx = 4 * k + e;  // value index i * E + mt
            v[e] = acc[0][idx % kE][idx / kE] * inv[0];
          }
          po[(wv * kE + k) * 64 + lane] = v;
        }
        if (lane < 16) pl[wv * 16 + lane] = m_run[0] + __builtin_amdgcn_logf(l_tot[0]);
        int prev = 0;
        if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        prev = __builtin_amdgcn_readfirstlane(prev);  // lane 0 is active (the unit's first row is real)
        if (prev != active - 1) return;
        float M = kNegInf;
        for (int w2 = 0; w2 < active; ++w2) M = fmaxf(M, pl[w2 * 16 + ln]);
        float L = 0.f;
#pragma unroll
        for (int mt = 0; mt < kE; ++mt) acc[0][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int w2 = 0; w2 < active; ++w2) {
          const float wt = __builtin_amdgcn_exp2f(pl[w2 * 16 + ln] - M);
          L += wt;
#pragma unroll
          for (int k = 0; k < kE; ++k) {
            const f32x4 v = po[(w2 * kE + k) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int idx = 4 * k + e;
              acc[0][idx % kE][idx / kE] += wt * v[e];
            }
          }
        }
        if (ngroups == 1) {
          write_out(0, 1.0f / L);
          return;
        }
        m_run[0] = M;
        l_tot[0] = L;
        inv[0] = 1.0f / L;
      }
      fused_merge<D, kR>(ms, unit, xr, ngroups, lane, acc, m_run, l_tot, inv, write_out, head_ok);
      return;
    }
  }
  if constexpr (kMode == kModeSplit) {
    static_assert(kR == 1, "the split path has one row group");
    // partials for merge_kernel: [B, Hq, P, D] and [B, Hq, P]
    const size_t row0 = qidx[0] * a.num_parts;  // qidx = b * Hq + hq
    float* o = a.ws_o + (row0 + p) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = (4 * q4 + i) * S::kE;
#pragma unroll
      for (int mt = 0; mt < S::kE; mt += 4)
        *reinterpret_cast<f32x4*>(o + d0 + mt) = f32x4{acc[0][mt][i] * inv[0], acc[0][mt + 1][i] * inv[0],
                                                       acc[0][mt + 2][i] * inv[0], acc[0][mt + 3][i] * inv[0]};
    }
    if (q4 == 0) a.ws_lse[row0 + p] = m_run[0] + __builtin_amdgcn_logf(l_tot[0]);
  } else {
    const size_t unit = (static_cast<size_t>(b) * a.num_kv_heads + j) * units_per_head + ui;
    fused_merge<D, kR>(MergeSpace{a.ws_o, a.ws_lse, a.counters, a.num_parts}, unit, p, nparts, lane, acc, m_run,
                       l_tot, inv, write_out, head_ok);
  }
}

// ---------------------------------------------------------------------------
// chunked prefill: K/V tiles shared through LDS (16-bit caches; 8-bit caches
// of head size 128)
// ---------------------------------------------------------------------------
// Prefill multiplies many query rows against the same keys, so it is bound by
// MFMA work and by the traffic that feeds the MFMAs, not by HBM bytes (page
// "KV Cache and Inference Optimization": prefill is compute-bound, decode
// memory-bound). A workgroup of kW waves, each holding kR groups of 16
// (token, head) rows of one KV head's chunk, walks the partition's key tiles
// kT at a time (one softmax step per kT tiles). The workgroup copies a step's
// tiles from the cache into LDS -- K in MFMA fragment order (fragment f, lane
// l at byte 1024 f + 16 l), V in the layout its MFMA operand reads want --
// with loads one step ahead and one barrier per step, and every wave runs its
// QK and PV MFMAs from there: a tile is fetched once per workgroup instead of
// once per wave. The register layouts, the online softmax and the 16-bit head
// + residual weights are those of the decode kernel's tile pairs.
//
// Workgroups are numbered so that consecutive numbers land on one XCD
// (workgroups are dealt to the XCDs round-robin by linear id) and the query
// tiles of one (sequence, KV head, partition), which read the same K/V, are
// consecutive: their tiles meet in that XCD's L2. The cache loads use the
// default cache policy for the same reason.
constexpr int kXcds = 8;  // MI355X: eight accelerator complex dies
#ifndef PKV_PREFILL_LDS
#define PKV_PREFILL_LDS 1
#endif
#ifndef PKV_PREFILL_LDS_ROWS
#define PKV_PREFILL_LDS_ROWS 2  // 16-row groups per wave
#endif
#ifndef PKV_PREFILL_TR
#define PKV_PREFILL_TR 1  // head size 128: V operands by transposing LDS reads
#endif
#ifndef PKV_PREFILL_TILES
#define PKV_PREFILL_TILES 4  // 16-row key tiles per softmax step (2 or 4)
#endif
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 4  // waves per workgroup (head size 128; 4 for 64)
#endif
constexpr int prefill_waves(int head_dim) { return head_dim == 64 ? 4 : PKV_PREFILL_WAVES; }

// kQ = 0: the caches hold T; kQFp8 / kQInt8: 8-bit codes (head size 128)
// with one fp32 scale per token row, staged in LDS as codes and converted
// exactly to T; the K scale multiplies the scores, the V scale the softmax
// weights. E4M3 codes (one packed convert per two) are converted by each wave
// as it reads them; INT8 codes (three instructions per two) once per step by
// the workgroup, a share per thread, into a second LDS area laid out as the
// 16-bit caches are.
template <typename T, int D, bool kNHD, int kW, int kR, int kT, int kQ>
__global__ __launch_bounds__(64 * kW) void prefill_lds_kernel(DecodeArgs a) {
  using S = Shape<T, D>;
  static_assert(sizeof(T) == 2, "16-bit queries and MFMA operands");
  static_assert(kT == 2 || kT == 4, "two or four tiles per step");
  constexpr bool kCodes = kQ != 0;
  constexpr bool kConvShared = kQ == kQInt8;          // converted once per step into ldsx
  constexpr bool kConvWave = kCodes && !kConvShared;  // converted by each wave from the codes
  static_assert(!kCodes || D == 128, "8-bit caches: head size 128");
  constexpr int kRowB = kCodes ? D : S::kRowBytes;    // bytes of a cache row
  constexpr int kNK = kRowB / 64;                     // K fragments (16 bytes per lane) per tile, as loaded
  constexpr int kKBytes = kT * kNK * 1024;            // K of a step's tiles, fragment order
  // 16-bit V as the MFMAs read it: head size 128 keeps each tile as four 1 KiB
  // blocks, block k holding rows k, 4+k, 8+k, 12+k (rows 4+k and 12+k with
  // their 128-byte halves swapped), each block 32 bytes after the previous one
  // ends, so the transposing reads of four rows 4*q4 + k at one column hit
  // distinct banks; head size 64 keeps plain row order (read with 16-byte
  // loads and shuffles). 8-bit codes are loaded in row order.
  constexpr bool kTrV = D == 128 && PKV_PREFILL_TR && !kConvWave;
  constexpr bool kTrLoad = kTrV && !kCodes;  // the loads place V in the block layout
  constexpr int kVBlock = 1024 + 32;
  constexpr int kVTileX = kTrV ? 4 * kVBlock : kTile * S::kRowBytes;
  constexpr int kVTileBytes = kCodes ? kTile * kRowB : kVTileX;
  constexpr int kVBytes = kT * kVTileBytes;  // V of a step's tiles, as loaded
  constexpr int kKBytesX = kT * S::kNK * 1024;  // INT8: the converted K (16-bit fragments), then V
  constexpr int kXBytes = kConvShared ? kKBytesX + kT * kVTileX : 16;
  constexpr int kSBytes = kCodes ? 2 * kT * kTile * 4 : 0;  // 8-bit: K, then V row scales of the tiles
  constexpr int kBuf = kKBytes + kVBytes + kSBytes;
  constexpr int kBufs = kT == 2 ? 3 : 2;  // LDS buffers: loads run kBufs - 1 steps ahead
  constexpr int kThreads = 64 * kW;
  constexpr int kKLoads = kKBytes / 16 / kThreads;  // 16-byte loads per thread per step
  constexpr int kVLoads = kT * kTile * kRowB / 16 / kThreads;
  constexpr int kSLoads = kCodes ? 2 * kT / kW : 0;  // 8-bit: scale rows per wave per step
  constexpr int kRowChunks = kRowB / 16;
  constexpr int kVTileChunks = kTile * kRowChunks;
  static_assert(kKLoads * 16 * kThreads == kKBytes && kVLoads * 16 * kThreads == kT * kTile * kRowB,
                "a step's tiles split evenly over the workgroup");
  static_assert(!kCodes || kSLoads * kW == 2 * kT, "scale rows split evenly over the waves");
  static_assert(!kTrLoad || kVLoads == kT, "one V block per wave per tile");
  static_assert(kVTileChunks % 64 == 0, "a wave's V chunks lie in one tile");
  // E4M3 V codes (row order, 128 bytes a row): the 16-byte chunks of row r of
  // the step's tile u are stored rotated by ((r >> 1) & 3) + 4 (u & 1), so the
  // transposing reads of a half-wave (8 rows of each tile of a pair, two
  // 8-byte halves of one chunk each) cover 256 distinct bytes of the bank space
  auto v8_rot = [](int row, int u) { return ((row >> 1) & 3) | ((u & 1) << 2); };
  // the LDS buffers as separate objects: the compiler then tracks which
  // buffer each cache -> LDS load writes and waits only for the right ones
  __shared__ __attribute__((aligned(16))) char lds0[kBuf];
  __shared__ __attribute__((aligned(16))) char lds1[kBuf];
  __shared__ __attribute__((aligned(16))) char lds2[kBufs > 2 ? kBuf : 16];
  __shared__ __attribute__((aligned(16))) char ldsx[kXBytes];
  // the partition's tile rows (-1: id outside the pool), then room for the
  // reads of whole steps past its end (their entries are not used)
  __shared__ __attribute__((aligned(16))) int trows[kMaxPrefillTiles + 8];

  // The lambdas below capture only locals: a lambda that referenced `a`
  // would take its address, and next to the cache -> LDS loads (which may
  // write memory as far as the compiler knows) the arguments would then be
  // copied to scratch and reloaded per lane.
  const char* const k_cache = a.k_cache;
  const char* const v_cache = a.v_cache;
  const char* const k_scales = a.k_scales;
  const char* const v_scales = a.v_scales;
  const int32_t* const tables = a.block_tables;
  char* const out = a.out;
  const int num_blocks = a.num_blocks;
  const int num_kv_heads = a.num_kv_heads;
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4;
  const int ln = lane & 15;

  // work unit (sequence b, KV head j, query tile ui, partition p), numbered
  // XCD-major: XCD x runs the x-th contiguous range of unit numbers
  const unsigned nwg = gridDim.x * gridDim.y * gridDim.z;
  const unsigned lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const unsigned xcd = lin % kXcds, per = nwg / kXcds, extra = nwg % kXcds;
  unsigned id = (xcd < extra ? xcd * (per + 1) : extra * (per + 1) + (xcd - extra) * per) + lin / kXcds;
  // query tiles in descending order: the later tiles of a chunk see more keys
  // (causal), and starting the longest workgroups first shortens the tail
  const int ui = a.q_tiles - 1 - static_cast<int>(id % static_cast<unsigned>(a.q_tiles));
  id /= static_cast<unsigned>(a.q_tiles);
  const int p = static_cast<int>(id % gridDim.x);
  id /= gridDim.x;
  const int j = static_cast<int>(id % static_cast<unsigned>(a.num_kv_heads));
  const int b = static_cast<int>(id / static_cast<unsigned>(a.num_kv_heads));

  // the chunk's query tokens are the last q_len of the sequence's n tokens
  const int cap = a.cap_tokens;
  int n = a.context_lens[b];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int q_tok0 = a.q_start[b];
  int q_len = a.q_start[b + 1] - q_tok0;
  q_len = q_len < 0 ? 0 : min(q_len, min(a.max_q_len, n));
  const int rows = q_len * a.group;
  const int first = n - q_len;  // position of the chunk's first token
  constexpr int kWgRows = kW * kR * kTile;
  const int wg_r0 = ui * kWgRows;
  if (wg_r0 >= rows) return;  // the whole workgroup: no rows
  // keys the workgroup reads: up to its last row's position
  const int n_wg = first + min(wg_r0 + kWgRows - 1, rows - 1) / a.group + 1;
  const int nblk_seq = (n_wg + kTile - 1) / kTile;
  const int nparts = (nblk_seq + a.pb_per_part - 1) / a.pb_per_part;
  if (p >= nparts) return;
  const int blk0 = p * a.pb_per_part;
  const int nblk = min(min(a.pb_per_part, kMaxPrefillTiles), nblk_seq - blk0);  // the host keeps pb in bounds

  // this wave's rows: kR groups of 16, row r = token r / g, head r % g
  const int r0 = wg_r0 + w * kR * kTile;
  const bool wave_rows = r0 < rows;
  const int n_w = wave_rows ? first + min(r0 + kR * kTile - 1, rows - 1) / a.group + 1 : 0;
  // the smallest key limit of the wave's rows (uniform: kept in a scalar register)
  const int min_limit = __builtin_amdgcn_readfirstlane(first + r0 / a.group + 1);
  int my_limit[kR];
  bool head_ok[kR];
  size_t qidx[kR];
  // Q as the B operand of chunk cc, in the d order of K: 16-bit caches keep
  // 16-byte chunk 4 cc + q4 of each row in lane (q4, .); 8-bit caches give
  // lane (q4, .) a row's codes q4 D/4 .. q4 D/4 + D/4 - 1, 8 per chunk
  u32x4 qv[kR][S::kNK];
#pragma unroll
  for (int rg = 0; rg < kR; ++rg) {
    const int r = r0 + rg * kTile + ln;
    head_ok[rg] = r < rows;
    const int tok = head_ok[rg] ? r / a.group : 0;
    const int hin = head_ok[rg] ? r - tok * a.group : 0;
    my_limit[rg] = head_ok[rg] ? first + tok + 1 : 0;
    qidx[rg] = (static_cast<size_t>(q_tok0) + tok) * a.num_heads + j * a.group + hin;
    const char* qrow = a.q + qidx[rg] * S::kRowBytes;
#pragma unroll
    for (int cc = 0; cc < S::kNK; ++cc) {
      const int off = kCodes ? q4 * (D / 2) + 16 * cc : (4 * cc + q4) * 16;
      qv[rg][cc] = head_ok[rg] ? *reinterpret_cast<const u32x4*>(qrow + off) : u32x4{0, 0, 0, 0};
    }
  }
  const float c = a.qk_scale;  // > 0: the host routes other scales to the one-wave kernel

  // first cache row of each of the partition's tiles, from the block table
  // into LDS once (a thread per tile), -1 for a block id outside the pool;
  // the barrier before the first loads publishes the table
  const size_t trow = static_cast<size_t>(b) * a.max_blocks;
  const int m = a.tiles_per_block;
  const int max_tiles = a.max_blocks * m;
  auto tile_row0 = [&](int lt) -> int {
    const int lb = lt / m;
    const int bid = tables[trow + lb];
    if (static_cast<unsigned>(bid) >= static_cast<unsigned>(num_blocks)) return -1;
    const int sub = lt - lb * m;
    return kNHD ? (bid * m + sub) * kTile * num_kv_heads + j : ((bid * num_kv_heads + j) * m + sub) * kTile;
  };
  // (a loop of fixed trip count: values computed in a loop whose exit
  // depends on the lane would count as divergent after it)
  static_assert(kMaxPrefillTiles % kThreads == 0, "table entries per thread");
#pragma unroll
  for (int i = 0; i < kMaxPrefillTiles / kThreads; ++i) {
    const int t = tid + kThreads * i;
    if (t < nblk) trows[t] = blk0 + t < max_tiles ? tile_row0(blk0 + t) : -1;
  }
  __syncthreads();
  const int rs = kRowB * (kNHD ? a.num_kv_heads : 1);  // bytes between a head's consecutive token rows
  const int ss = kNHD ? 4 * a.num_kv_heads : 4;        // 8-bit: bytes between their scales
  // first cache row of each of step s's tiles and their rows to fetch, from
  // one LDS read of the step's table entries: 0 past the partition end or for
  // an id outside the pool (nothing is read then)
  static_assert(kT * (kMaxPrefillTiles / kT + 2) <= kMaxPrefillTiles + 8, "table reads of steps past the end");
  auto step_src = [&](int s, size_t (&row)[kT], int (&valid)[kT]) __attribute__((always_inline)) {
    int e[kT];
    if constexpr (kT == 4) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(trows + kT * s);
      for (int u = 0; u < kT; ++u) e[u] = static_cast<int>(x[u]);
    } else {
      const u32x2 x = *reinterpret_cast<const u32x2*>(trows + kT * s);
      for (int u = 0; u < kT; ++u) e[u] = static_cast<int>(x[u]);
    }
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      const int t = kT * s + u;
      const int r = __builtin_amdgcn_readfirstlane(e[u]);
      const bool ok = t < nblk && r >= 0;
      valid[u] = ok ? min(kTile, n_wg - (blk0 + t) * kTile) : 0;
      row[u] = ok ? static_cast<size_t>(r) : 0;
    }
  };

  const int nsteps = (nblk + kT - 1) / kT;  // steps of kT tiles
  // cache -> LDS for the kT tiles of step s, straight into LDS buffer `dst`
  // (buffer loads with the LDS flag: lane l's 16 bytes land at M0 + 16 l);
  // each tile's valid row count goes to `valid` for the step's softmax
  auto fetch = [&](int s, char* dst, int (&valid)[kT]) __attribute__((always_inline)) {
    __amdgpu_buffer_rsrc_t rk[kT], rv[kT];
    size_t row[kT];
    step_src(s, row, valid);
#pragma unroll
    for (int u = 0; u < kT; ++u) {
      rk[u] = tile_rsrc(k_cache + row[u] * kRowB, valid[u] * rs);
      rv[u] = tile_rsrc(v_cache + row[u] * kRowB, valid[u] * rs);
    }
    // the tile of a wave's i-th load: t0, or t0 + 1 for the upper half of the
    // waves where one tile's K (or V) is half of what the workgroup loads at once
    constexpr bool kKHalf = kNK < kW, kVHalf = kVTileChunks < 64 * kW;
    static_assert(kNK == kW || 2 * kNK == kW, "four waves, 64- or 128-element rows");
    static_assert(kVTileChunks == 64 * kW || 2 * kVTileChunks == 64 * kW, "V chunks per tile");
    auto pick = [&](const __amdgpu_buffer_rsrc_t (&r)[kT], int t0, bool half) __attribute__((always_inline)) {
      return half && w >= kW / 2 ? r[t0 + 1] : r[t0];
    };
    // Every resource reaches the LDS-load builtin as a named local: given a
    // temporary or an array element, the host compilation pass drops the
    // kernel's launch stub (the library then fails to load).
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      // fragment f = w + kW i of the step: tile f / kNK, chunk group cg = f % kNK;
      // lane (q4, ln) takes token ln's 16-byte chunk 4 cg + q4 (8-bit: the
      // chunk at byte q4 D/4 + 16 cg)
      const int f = w + kW * i;
      const int cg = f % kNK;
      const int col = kCodes ? q4 * (D / 4) + 16 * cg : (4 * cg + q4) * 16;
      const __amdgpu_buffer_rsrc_t r = pick(rk, kW * i / kNK, kKHalf);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(dst + f * 1024), 16, ln * rs + col, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      if constexpr (kTrLoad) {
        // tile i, block w: lane l fills row 4 (l / 16) + w, 16-byte chunk l % 16
        // of the block, taking the row's chunk (l % 16) ^ 8 for odd l / 16
        const int row = 4 * (lane >> 4) + w, col = (lane & 15) ^ (((lane >> 4) & 1) << 3);
        const __amdgpu_buffer_rsrc_t r = rv[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(dst + kKBytes + i * kVTileBytes + w * kVBlock), 16,
                                                 row * rs + col * 16, 0, 0, 0);
      } else {
        const int cw = 64 * w + kThreads * i;  // the wave's first V chunk of the step
        const int u = cw / kVTileChunks;
        const int ch = cw - u * kVTileChunks + lane;
        const int row = ch / kRowChunks;
        int col = ch - (ch / kRowChunks) * kRowChunks;
        if constexpr (kConvWave) col ^= v8_rot(row, u);  // LDS chunk c of the row holds its chunk c ^ rot
        const __amdgpu_buffer_rsrc_t r = pick(rv, kThreads * i / kVTileChunks, kVHalf);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(dst + kKBytes + cw * 16), 16, row * rs + col * 16, 0, 0,
                                                 0);
      }
    }
    if constexpr (kCodes) {
      // scale row j = w + kW i of the step: K (j even) or V scales of tile
      // j / 2, 4 bytes per lane from the first 16 lanes (the rows past the
      // tile's valid count read as zero)
#pragma unroll
      for (int i = 0; i < kSLoads; ++i) {
        const int jj = w + kW * i, tile = jj >> 1;
        const __amdgpu_buffer_rsrc_t r =
            tile_rsrc(((jj & 1) ? v_scales : k_scales) + row[tile] * 4, valid[tile] * ss);
        if (lane < kTile)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              r, lds_ptr(dst + kKBytes + kVBytes + (jj & 1) * (kT * kTile * 4) + tile * (kTile * 4)), 4, lane * ss,
              0, 0, 0);
      }
    }
  };
  // every wave's loads into the next buffer have landed once each wave has
  // drained its own (all but those of the steps further ahead) and the
  // barrier is passed
  constexpr int kLoads = kKLoads + kVLoads + kSLoads;
  constexpr int kNewer = (kBufs - 2) * kLoads;  // loads that may stay in flight
  static_assert(kNewer < 16, "vmcnt field");
  auto sync_step = [&]() __attribute__((always_inline)) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xF70 | kNewer);  // vmcnt <= kNewer (expcnt, lgkmcnt: no wait)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  f32x4 acc[kR][S::kE];
  float m_run[kR];  // running max of scaled scores (log2 units)
  float l_run[kR];  // this lane's share of the running denominator
#pragma unroll
  for (int rg = 0; rg < kR; ++rg) {
#pragma unroll
    for (int mt = 0; mt < S::kE; ++mt) acc[rg][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rg] = kNegInf;
    l_run[rg] = 0.f;
  }

  // QK^T of step s (its 16-bit K fragments at kl) for every row group and
  // tile; 8-bit: times the keys' K scales (at sl)
  auto scores = [&](const char* kl, const char* sl, f32x4 (&sc)[kR][kT]) __attribute__((always_inline)) {
#pragma unroll
    for (int rg = 0; rg < kR; ++rg)
#pragma unroll
      for (int u = 0; u < kT; ++u) sc[rg][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kConvWave) {
#pragma unroll
      for (int cc = 0; cc < kNK; ++cc) {
        // 16 codes per lane: 16-bit chunks 2 cc (bytes 0..7) and 2 cc + 1
        u32x4 k0[kT], k1[kT];
#pragma unroll
        for (int u = 0; u < kT; ++u) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(kl + (u * kNK + cc) * 1024 + lane * 16);
          const u32x2 x0 = codes4_to_16<kQ, T>(raw[0]), x1 = codes4_to_16<kQ, T>(raw[1]);
          const u32x2 x2 = codes4_to_16<kQ, T>(raw[2]), x3 = codes4_to_16<kQ, T>(raw[3]);
          k0[u] = u32x4{x0[0], x0[1], x1[0], x1[1]};
          k1[u] = u32x4{x2[0], x2[1], x3[0], x3[1]};
        }
#pragma unroll
        for (int rg = 0; rg < kR; ++rg)
#pragma unroll
          for (int u = 0; u < kT; ++u) sc[rg][u] = mfma_qk16<T>(k0[u], qv[rg][2 * cc], sc[rg][u]);
#pragma unroll
        for (int rg = 0; rg < kR; ++rg)
#pragma unroll
          for (int u = 0; u < kT; ++u) sc[rg][u] = mfma_qk16<T>(k1[u], qv[rg][2 * cc + 1], sc[rg][u]);
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < S::kNK; ++cc) {
        u32x4 kf[kT];
#pragma unroll
        for (int u = 0; u < kT; ++u)
          kf[u] = *reinterpret_cast<const u32x4*>(kl + (u * S::kNK + cc) * 1024 + lane * 16);
#pragma unroll
        for (int rg = 0; rg < kR; ++rg)
#pragma unroll
          for (int u = 0; u < kT; ++u) sc[rg][u] = mfma_qk16<T>(kf[u], qv[rg][cc], sc[rg][u]);
      }
    }
    if constexpr (kCodes) {  // the K scales of this lane's keys 4*q4 + i
#pragma unroll
      for (int u = 0; u < kT; ++u) {
        const f32x4 ksv = *reinterpret_cast<const f32x4*>(sl + u * (kTile * 4) + q4 * 16);
#pragma unroll
        for (int rg = 0; rg < kR; ++rg)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[rg][u][i] *= ksv[i];
      }
    }
  };
  // online-softmax step and PV products of step s (its V rows at vl); the
  // scores are raw (the scale c = qk_scale > 0 is applied inside the
  // exponent: max(c s) = c max(s)) and masked keys score -inf
  auto attend = [&](const char* vl, int s, f32x4 (&sc)[kR][kT], const int (&valid)[kT], const char* sl)
                    __attribute__((always_inline)) {
    const int key0 = (blk0 + kT * s) * kTile;
    // rows past a tile's valid count were not fetched (they read as zero);
    // keys past a row's position are masked: lane (q4, .) keeps its rows
    // 4*q4 + i below both limits. The tests are wave-uniform, and a step of
    // full tiles below every row's limit (all but a partition's last ones)
    // skips them with one.
    int vmin = kTile;
#pragma unroll
    for (int u = 0; u < kT; ++u) vmin = min(vmin, __builtin_amdgcn_readfirstlane(valid[u]));
    if (vmin < kTile || key0 + kT * kTile > min_limit) {
#pragma unroll
      for (int rg = 0; rg < kR; ++rg)
#pragma unroll
        for (int u = 0; u < kT; ++u) {
          const int key = key0 + u * kTile;
          if (__builtin_amdgcn_readfirstlane(valid[u]) < kTile || key + kTile > min_limit) {
            const int lim = min(valid[u], my_limit[rg] - key) - 4 * q4;
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[rg][u][i] = i < lim ? sc[rg][u][i] : kNegInf;
          }
        }
    }
    float mx[kR];
    bool grow_any = false;
#pragma unroll
    for (int rg = 0; rg < kR; ++rg) {
      float m4 = kNegInf;
#pragma unroll
      for (int u = 0; u < kT; ++u)
        m4 = fmax_nan(m4, fmax_nan(fmax_nan(sc[rg][u][0], sc[rg][u][1]), fmax_nan(sc[rg][u][2], sc[rg][u][3])));
      mx[rg] = quarter_max(m4) * c;  // -inf stays -inf (c > 0)
      grow_any |= mx[rg] > m_run[rg] + kRescaleSlack;
    }
    // one wave-uniform rescale decision for all row groups of the step
    if (__builtin_amdgcn_ballot_w64(grow_any)) {
#pragma unroll
      for (int rg = 0; rg < kR; ++rg) {
        const bool grow = mx[rg] > m_run[rg] + kRescaleSlack;
        const float m_new = grow ? mx[rg] : m_run[rg];
        const float alpha = m_run[rg] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run[rg] - m_new);
#pragma unroll
        for (int mt = 0; mt < S::kE; ++mt) acc[rg][mt] *= alpha;
        l_run[rg] *= alpha;
        m_run[rg] = m_new;
      }
    }
    // weights as 16-bit head + residual, per pair of tiles: the MFMA's K index
    // runs over tile 2pp's rows 4*q4 .. 4*q4+3, then tile 2pp+1's
    u32x4 pw_hi[kR][kT / 2], pw_lo[kR][kT / 2];
#pragma unroll
    for (int rg = 0; rg < kR; ++rg) {
      const float m_use = m_run[rg] == kNegInf ? 0.f : m_run[rg];
      float lsum = 0.f;
#pragma unroll
      for (int pp = 0; pp < kT / 2; ++pp) {
        float pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[rg][2 * pp + i / 4][i % 4], c, -m_use));
          lsum += pr[i];
        }
        if constexpr (kCodes) {  // the V scale rides on the weight
          const char* vsl = sl + kT * kTile * 4;
          const f32x4 va = *reinterpret_cast<const f32x4*>(vsl + (2 * pp) * (kTile * 4) + q4 * 16);
          const f32x4 vb = *reinterpret_cast<const f32x4*>(vsl + (2 * pp + 1) * (kTile * 4) + q4 * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pr[i] *= va[i];
            pr[4 + i] *= vb[i];
          }
        }
        unsigned hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split16_pair<T>(pr[2 * i], pr[2 * i + 1], hi[i], lo[i]);
        pw_hi[rg][pp] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        pw_lo[rg][pp] = u32x4{lo[0], lo[1], lo[2], lo[3]};
      }
      l_run[rg] += lsum;
    }
#pragma unroll
    for (int pp = 0; pp < kT / 2; ++pp) {
      if constexpr (kTrV) {
        // Transposing reads (ds_read_b64_tr_b16): in each quarter-wave, lane
        // s = 4k + a names 8 bytes of row 4*q4 + k at column 16 mt + 4a, and
        // lane r receives the four rows' values at column 16 mt + r -- the A
        // operand of output block mt (rows d = 16 mt + r) for this quarter's keys.
        // Odd q4 rows hold their two 128-byte halves swapped (column block mt
        // at mt ^ 4), so the two quarter-waves of each half-wave read
        // different 128-byte bank ranges.
        const int sk = ln >> 2, sa = ln & 3;
        const int swz = (q4 & 1) * 128;
        const char* base = vl + sk * kVBlock + q4 * S::kRowBytes + sa * 8;
        const char* base_lo = base + swz;  // column blocks 0..3
        const char* base_hi = base - swz;  // column blocks 4..7
#pragma unroll
        for (int mt = 0; mt < S::kE; ++mt) {
          const char* bm = (mt < 4 ? base_lo : base_hi) + mt * 32;
          const auto x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(bm + (2 * pp) * kVTileX));
          const auto y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(bm + (2 * pp + 1) * kVTileX));
          const u32x2 xa = __builtin_bit_cast(u32x2, x), yb = __builtin_bit_cast(u32x2, y);
          const u32x4 av = {xa[0], xa[1], yb[0], yb[1]};
#pragma unroll
          for (int rg = 0; rg < kR; ++rg) {
            acc[rg][mt] = mfma_qk16<T>(av, pw_hi[rg][pp], acc[rg][mt]);
            acc[rg][mt] = mfma_qk16<T>(av, pw_lo[rg][pp], acc[rg][mt]);
          }
        }
        continue;
      }
      if constexpr (kConvWave) {
        // Transposing 8-bit reads (ds_read_b64_tr_b8): in each quarter-wave,
        // lane s = 2e + h names 8 codes of key e (rows 4*q4 + e of tile 2pp for
        // e < 4, rows 4*q4 + e - 4 of tile 2pp+1) at columns 16 mt + 8h, and
        // lane i receives byte (i & 7) of lanes 2e + (i >> 3), e = 0..7: the
        // eight keys' codes at column 16 mt + i, which converted in order are
        // the A operand of output block mt (rows d = 16 mt + i).
        const int e = ln >> 1, h = ln & 1;
        const int tu = 2 * pp + (e >> 2), row = 4 * q4 + (e & 3);
        const char* rb = vl + (tu * kTile + row) * kRowB + 8 * h;
        const int rot = v8_rot(row, tu);
#pragma unroll
        for (int mt = 0; mt < S::kE; ++mt) {
          const auto x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(rb + (mt ^ rot) * 16));
          const u32x2 c2 = __builtin_bit_cast(u32x2, x);
          const u32x2 lo = codes4_to_16<kQ, T>(c2[0]), hi = codes4_to_16<kQ, T>(c2[1]);
          const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int rg = 0; rg < kR; ++rg) {
            acc[rg][mt] = mfma_qk16<T>(av, pw_hi[rg][pp], acc[rg][mt]);
            acc[rg][mt] = mfma_qk16<T>(av, pw_lo[rg][pp], acc[rg][mt]);
          }
        }
        continue;
      }
      // V rows 4*q4 + i of tiles 2pp and 2pp+1, this lane's E elements,
      // packed into the A operand of each output block mt
      unsigned v_a[4][S::kVDW], v_b[4][S::kVDW];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* ra = vl + (2 * pp * kTile + 4 * q4 + i) * S::kRowBytes + ln * S::kE * 2;
        const char* rb = ra + kTile * S::kRowBytes;
        if constexpr (S::kVDW == 4) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(ra);
          const u32x4 y = *reinterpret_cast<const u32x4*>(rb);
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            v_a[i][d] = x[d];
            v_b[i][d] = y[d];
          }
        } else {
          static_assert(S::kVDW == 2, "16-bit rows of 64 or 128 elements");
          const u32x2 x = *reinterpret_cast<const u32x2*>(ra);
          const u32x2 y = *reinterpret_cast<const u32x2*>(rb);
          v_a[i][0] = x[0];
          v_a[i][1] = x[1];
          v_b[i][0] = y[0];
          v_b[i][1] = y[1];
        }
      }
#pragma unroll
      for (int mt = 0; mt < S::kE; ++mt) {
        const unsigned sel = (mt & 1) ? 0x07060302u : 0x05040100u;
        const u32x4 av = {__builtin_amdgcn_perm(v_a[1][mt >> 1], v_a[0][mt >> 1], sel),
                          __builtin_amdgcn_perm(v_a[3][mt >> 1], v_a[2][mt >> 1], sel),
                          __builtin_amdgcn_perm(v_b[1][mt >> 1], v_b[0][mt >> 1], sel),
                          __builtin_amdgcn_perm(v_b[3][mt >> 1], v_b[2][mt >> 1], sel)};
#pragma unroll
        for (int rg = 0; rg < kR; ++rg) {
          acc[rg][mt] = mfma_qk16<T>(av, pw_hi[rg][pp], acc[rg][mt]);
          acc[rg][mt] = mfma_qk16<T>(av, pw_lo[rg][pp], acc[rg][mt]);
        }
      }
    }
  };

  // INT8: the codes of a step (buffer cb) -> T in ldsx, 16 codes per thread
  // and pass: K fragment f, lane l -> 16-bit fragments 2 (f % kNK) and
  // 2 (f % kNK) + 1 of its tile, lane l (bytes 0..7, then 8..15); V row r,
  // codes 16 c .. 16 c + 15 -> elements 16 c .. 16 c + 15 of row r in the
  // block layout. Every byte the MFMAs read is rewritten each step.
  auto convert = [&](const char* cb) __attribute__((always_inline)) {
    constexpr int kKChunks = kT * kNK * 64, kVChunks = kT * kVTileChunks;
    static_assert(kKChunks % kThreads == 0 && kVChunks % kThreads == 0, "conversion passes");
#pragma unroll
    for (int i = 0; i < kKChunks / kThreads; ++i) {
      const int g = tid + kThreads * i;
      const int f = g >> 6, l = g & 63;
      const int u = f / kNK, cg = f - u * kNK;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(cb + g * 16);
      const u32x2 x0 = codes4_to_16<kQ, T>(raw[0]), x1 = codes4_to_16<kQ, T>(raw[1]);
      const u32x2 x2 = codes4_to_16<kQ, T>(raw[2]), x3 = codes4_to_16<kQ, T>(raw[3]);
      char* dk = ldsx + ((u * S::kNK + 2 * cg) * 64 + l) * 16;
      *reinterpret_cast<u32x4*>(dk) = u32x4{x0[0], x0[1], x1[0], x1[1]};
      *reinterpret_cast<u32x4*>(dk + 1024) = u32x4{x2[0], x2[1], x3[0], x3[1]};
    }
#pragma unroll
    for (int i = 0; i < kVChunks / kThreads; ++i) {
      const int g = tid + kThreads * i;
      const int u = g / kVTileChunks, ch = g - u * kVTileChunks;
      const int row = ch / kRowChunks, col = ch - row * kRowChunks;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(cb + kKBytes + g * 16);
      const u32x2 x0 = codes4_to_16<kQ, T>(raw[0]), x1 = codes4_to_16<kQ, T>(raw[1]);
      const u32x2 x2 = codes4_to_16<kQ, T>(raw[2]), x3 = codes4_to_16<kQ, T>(raw[3]);
      const int at = kTrV ? (row & 3) * kVBlock + (row >> 2) * S::kRowBytes + ((col * 32) ^ (((row >> 2) & 1) * 128))
                          : row * S::kRowBytes + col * 32;
      char* dv = ldsx + kKBytesX + u * kVTileX + at;
      *reinterpret_cast<u32x4*>(dv) = u32x4{x0[0], x0[1], x1[0], x1[1]};
      *reinterpret_cast<u32x4*>(dv + 16) = u32x4{x2[0], x2[1], x3[0], x3[1]};
    }
  };
  // every wave's conversion writes have landed once each wave has drained its
  // own LDS operations and the barrier is passed (the cache loads in flight
  // are not waited for)
  auto sync_lds = [&]() __attribute__((always_inline)) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0 (vmcnt, expcnt: no wait)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  // kBufs buffers, loads kBufs - 1 steps ahead: step s consumes buffer
  // s % kBufs while the next steps load; its barrier makes step s+1 visible
  // and frees buffer s % kBufs. Past the partition end the loads fetch nothing.
  char* const bufs[3] = {lds0, lds1, lds2};
  int valid[kBufs][kT];  // valid rows of the tiles in each buffer
#pragma unroll
  for (int u = 0; u < kBufs - 1; ++u) fetch(u, bufs[u], valid[u]);
  sync_step();
  auto step = [&](int s, int cur, int ahead) __attribute__((always_inline)) {
    fetch(s + kBufs - 1, bufs[ahead], valid[ahead]);
    if constexpr (kConvShared) {  // every wave takes part, with rows or not
      convert(bufs[cur]);
      sync_lds();
    }
    if (wave_rows && (blk0 + kT * s) * kTile < n_w) {  // wave-uniform: some key of the step is visible
      f32x4 sc[kR][kT];
      const char* xb = kConvShared ? ldsx : bufs[cur];
      const char* sl = bufs[cur] + kKBytes + kVBytes;  // 8-bit: the row scales
      scores(xb, sl, sc);
      attend(xb + (kConvShared ? kKBytesX : kKBytes), s, sc, valid[cur], sl);
    }
    sync_step();
  };
  for (int s0 = 0; s0 < nsteps; s0 += kBufs) {
#pragma unroll
    for (int u = 0; u < kBufs; ++u)
      if (u == 0 || s0 + u < nsteps) step(s0 + u, u, (u + kBufs - 1) % kBufs);
  }
  __builtin_amdgcn_s_waitcnt(0xF70);  // no load into LDS outlives the workgroup
  if (!wave_rows) return;

  float l_tot[kR], inv[kR];
#pragma unroll
  for (int rg = 0; rg < kR; ++rg) {
    l_tot[rg] = l_run[rg] + xor_shuffle(l_run[rg], 16);
    l_tot[rg] += xor_shuffle(l_tot[rg], 32);
    inv[rg] = l_tot[rg] > 0.f ? 1.0f / l_tot[rg] : 0.f;
  }
  // this lane's 4 x E output values of row group rg: d = 16 mt + 4*q4 + i
  // (transposed V reads, 16- or 8-bit), else d = (4*q4 + i) * E + mt
  auto write_out = [&](int rg, float scale_by) {
    if (!head_ok[rg]) return;
    char* orow = out + qidx[rg] * S::kRowBytes;
    if constexpr (kTrV || kConvWave) {
#pragma unroll
      for (int mt = 0; mt < S::kE; ++mt) {
        const u32x2 wv = {to_bits16<T>(acc[rg][mt][0] * scale_by) | (to_bits16<T>(acc[rg][mt][1] * scale_by) << 16),
                          to_bits16<T>(acc[rg][mt][2] * scale_by) | (to_bits16<T>(acc[rg][mt][3] * scale_by) << 16)};
        *reinterpret_cast<u32x2*>(orow + (16 * mt + 4 * q4) * 2) = wv;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        unsigned wv[S::kVDW];
#pragma unroll
        for (int mt = 0; mt < S::kE; mt += 2)
          wv[mt >> 1] = to_bits16<T>(acc[rg][mt][i] * scale_by) | (to_bits16<T>(acc[rg][mt + 1][i] * scale_by) << 16);
        store_dwords<S::kVDW>(orow + (4 * q4 + i) * S::kE * 2, wv);
      }
    }
  };
  if (nparts == 1) {
#pragma unroll
    for (int rg = 0; rg < kR; ++rg) write_out(rg, inv[rg]);
    return;
  }
  const size_t unit = ((static_cast<size_t>(b) * a.num_kv_heads + j) * a.q_tiles + ui) * kW + w;  // one per wave
  fused_merge<D, kR>(MergeSpace{a.ws_o, a.ws_lse, a.counters, a.num_parts}, unit, p, nparts, lane, acc, m_run, l_tot,
                     inv, write_out, head_ok);
}

// ---------------------------------------------------------------------------
// log-sum-exp merge of partitions: one wave per (sequence, query head)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, int num_seqs) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= num_seqs * a.num_heads) return;
  const int b = wave / a.num_heads;
  const int hq = wave - b * a.num_heads;
  const int cap = a.cap_tokens;
  int n = a.context_lens[b];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int nblk_seq = (n + kTile - 1) / kTile;
  const int nparts = nblk_seq == 0 ? 1 : (nblk_seq + a.pb_per_part - 1) / a.pb_per_part;
  if (nparts == 1) return;  // the partition kernel wrote this row directly
  const size_t row0 = (static_cast<size_t>(b) * a.num_heads + hq) * a.num_parts;
  float M = kNegInf;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.ws_lse[row0 + p]);
  constexpr int kPer = D / 64;  // elements per lane
  float accum[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) accum[e] = 0.f;
  float L = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = __builtin_amdgcn_exp2f(a.ws_lse[row0 + p] - M);
    L += w;
    const float* o = a.ws_o + (row0 + p) * D + lane * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) accum[e] += w * o[e];
  }
  const float inv = 1.0f / L;
  char* orow = a.out + (static_cast<size_t>(b) * a.num_heads + hq) * D * sizeof(T);
  if constexpr (sizeof(T) == 2) {
    unsigned short* dst = reinterpret_cast<unsigned short*>(orow) + lane * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) dst[e] = static_cast<unsigned short>(to_bits16<T>(accum[e] * inv));
  } else {
    float* dst = reinterpret_cast<float*>(orow) + lane * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) dst[e] = accum[e] * inv;
  }
}

// ---------------------------------------------------------------------------
// copy-on-write: whole blocks of up to four cache tensors, one workgroup per
// (pair, tensor), 16 bytes per thread per step with four copies in flight
// ---------------------------------------------------------------------------
struct CopyArgs {
  char* base[4];
  int64_t bytes[4];  // per block, multiple of 16
};

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a, const int32_t* __restrict__ pairs,
                                                          int32_t num_blocks) {
  const int32_t src = pairs[2 * static_cast<int64_t>(blockIdx.x)];
  const int32_t dst = pairs[2 * static_cast<int64_t>(blockIdx.x) + 1];
  if (src == dst || static_cast<unsigned>(src) >= static_cast<unsigned>(num_blocks) ||
      static_cast<unsigned>(dst) >= static_cast<unsigned>(num_blocks))
    return;
  const unsigned c = blockIdx.y;  // select, not index: keeps the arguments out of scratch
  char* base = c == 0 ? a.base[0] : c == 1 ? a.base[1] : c == 2 ? a.base[2] : a.base[3];
  const int64_t nb = c == 0 ? a.bytes[0] : c == 1 ? a.bytes[1] : c == 2 ? a.bytes[2] : a.bytes[3];
  const u32x4* s = reinterpret_cast<const u32x4*>(base + static_cast<int64_t>(src) * nb);
  u32x4* d = reinterpret_cast<u32x4*>(base + static_cast<int64_t>(dst) * nb);
  const int64_t chunks = nb / 16;
  int64_t i = threadIdx.x;
  for (; i + 3 * 256 < chunks; i += 4 * 256) {
    const u32x4 x0 = s[i], x1 = s[i + 256], x2 = s[i + 512], x3 = s[i + 768];
    d[i] = x0;
    d[i + 256] = x1;
    d[i + 512] = x2;
    d[i + 768] = x3;
  }
  for (; i < chunks; i += 256) d[i] = s[i];
}

// ---------------------------------------------------------------------------
// Read ceiling of the decode access pattern (a measurement kernel): the same
// partitions, block-table lookups and bounded nontemporal tile loads as a
// decode launch over the same cache, in the split decode launch's workgroups
// (consecutive KV heads of one partition) and XCD rotation, with nothing
// computed but an XOR of the loaded words (stored to `sink`, one word per lane
// and wave, so the loads stay live). Whatever rate this reaches is what the
// memory system gives for these tiles; the decode kernels are measured
// against it.
// ---------------------------------------------------------------------------
struct StreamArgs {
  const char* k;
  const char* v;
  const char* ks;  // per-row fp32 scales (8-bit caches), or null
  const char* vs;
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint32_t* sink;  // [B, Hkv, P, 64]
  int32_t max_blocks;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t tiles_per_block;  // block_size / 16
  int32_t pb_per_part;      // 16-row tiles per partition (<= 128)
  int32_t num_parts;
  int32_t cap_tokens;
  int32_t row_bytes;   // one head's token row
  int32_t nhd;         // token-major blocks: a head's rows num_kv_heads * row_bytes apart
};

template <int NC, bool kScales>  // NC: 16-byte chunks per lane per 16-row tile (row_bytes / 64)
__global__ __launch_bounds__(64 * PKV_DECODE_WAVES) void stream_tiles_kernel(StreamArgs a) {
  constexpr int kRowB = NC * 64;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int p = PKV_XCD_ROTATE ? static_cast<int>((blockIdx.x + blockIdx.y + gridDim.y * blockIdx.z) % gridDim.x)
                               : static_cast<int>(blockIdx.x);
  const int j = static_cast<int>(blockIdx.y) * static_cast<int>(blockDim.x >> 6) +
                __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int b = blockIdx.z;
  const int cap = a.cap_tokens;
  // the same start as the decode kernels: length and table entries requested together
  int n = a.context_lens[b];
  const int blk0 = p * a.pb_per_part;
  const size_t trow = static_cast<size_t>(b) * a.max_blocks;
  const int m = a.tiles_per_block;
  const int max_tiles = a.max_blocks * m;
  auto table_id = [&](int lt) __attribute__((always_inline)) -> int {
    const int lbc = min(lt, max_tiles - 1) / m;
    const int id = a.block_tables[trow + lbc];
    return lt < max_tiles ? id : -1;
  };
  auto row_of = [&](int id, int lt) __attribute__((always_inline)) -> int {
    if (static_cast<unsigned>(id) >= static_cast<unsigned>(a.num_blocks)) return -1;
    const int sub = lt - (lt / m) * m;
    return a.nhd ? (id * m + sub) * kTile * a.num_kv_heads + j : ((id * a.num_kv_heads + j) * m + sub) * kTile;
  };
  const int raw0 = table_id(blk0 + lane);
  const int id0 = lane < a.pb_per_part ? raw0 : -1;
  int id1 = -1;
  if (a.pb_per_part > 64) {  // wave-uniform
    const int raw1 = table_id(blk0 + 64 + lane);
    id1 = 64 + lane < a.pb_per_part ? raw1 : -1;
  }
  __builtin_amdgcn_sched_barrier(0);  // the length and table loads are issued before any wait on them
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int ntiles = (n + kTile - 1) / kTile;
  const int nparts = ntiles == 0 ? 1 : (ntiles + a.pb_per_part - 1) / a.pb_per_part;
  if (p >= nparts) return;
  const int nblk = min(a.pb_per_part, ntiles - blk0);
  const int my_r0 = row_of(id0, blk0 + lane), my_r02 = row_of(id1, blk0 + 64 + lane);
  const int rs = a.nhd ? kRowB * a.num_kv_heads : kRowB;  // bytes between a head's consecutive rows
  const int ss = a.nhd ? 4 * a.num_kv_heads : 4;          // the same for the scales
  constexpr int kAhead = 3, kRing = kAhead + 1;
  u32x4 rk[kRing][NC], rv[kRing][NC], rks[kRing], rvs[kRing];
  auto issue = [&](int u, int t) __attribute__((always_inline)) {  // u: ring slot (compile-time after unrolling)
    const int tt = min(t, 127);
    const int r0 = tt < 64 ? __builtin_amdgcn_readlane(my_r0, tt & 63) : __builtin_amdgcn_readlane(my_r02, tt & 63);
    const bool ok = t < nblk && r0 >= 0;
    const int rows = ok ? min(kTile, n - (blk0 + t) * kTile) : 0;
    const size_t row0 = ok ? static_cast<size_t>(r0) : 0;
    const __amdgpu_buffer_rsrc_t rk_ = tile_rsrc(a.k + row0 * kRowB, rows * rs);
    const __amdgpu_buffer_rsrc_t rv_ = tile_rsrc(a.v + row0 * kRowB, rows * rs);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int byte = (c * 64 + lane) * 16;  // byte of the tile's packed [16, row] bytes
      const int off = (byte / kRowB) * rs + byte % kRowB;
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rk_, off, 0, kCacheNT);
      const auto y = __builtin_amdgcn_raw_buffer_load_b128(rv_, off, 0, kCacheNT);
      rk[u][c] = u32x4{x[0], x[1], x[2], x[3]};
      rv[u][c] = u32x4{y[0], y[1], y[2], y[3]};
    }
    if constexpr (kScales) {
      const __amdgpu_buffer_rsrc_t rks_ = tile_rsrc(a.ks + row0 * 4, rows * ss);
      const __amdgpu_buffer_rsrc_t rvs_ = tile_rsrc(a.vs + row0 * 4, rows * ss);
      if (a.nhd) {  // one row's scale per lane of the first 16
        rks[u] = u32x4{__builtin_amdgcn_raw_buffer_load_b32(rks_, (lane & 15) * ss, 0, kCacheNT), 0u, 0u, 0u};
        rvs[u] = u32x4{__builtin_amdgcn_raw_buffer_load_b32(rvs_, (lane & 15) * ss, 0, kCacheNT), 0u, 0u, 0u};
      } else {  // the tile's 16 scales, as the decode kernel reads them (16 bytes per quarter-wave)
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rks_, 16 * (lane >> 4), 0, kCacheNT);
        const auto y = __builtin_amdgcn_raw_buffer_load_b128(rvs_, 16 * (lane >> 4), 0, kCacheNT);
        rks[u] = u32x4{x[0], x[1], x[2], x[3]};
        rvs[u] = u32x4{y[0], y[1], y[2], y[3]};
      }
    }
  };
  u32x4 acc = {0u, 0u, 0u, 0u};
  auto consume = [&](int u) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NC; ++c) acc ^= rk[u][c] ^ rv[u][c];
    if constexpr (kScales) acc ^= rks[u] ^ rvs[u];
  };
#pragma unroll
  for (int u = 0; u < kAhead; ++u) issue(u, u);
  for (int t0 = 0; t0 < nblk; t0 += kRing) {
#pragma unroll
    for (int uu = 0; uu < kRing; ++uu) {
      issue((uu + kAhead) % kRing, t0 + uu + kAhead);
      __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before any wait below
      if (t0 + uu < nblk) consume(uu);
    }
  }
  const size_t w = ((static_cast<size_t>(b) * a.num_kv_heads + j) * a.num_parts + p) * 64 + lane;
  a.sink[w] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// ---------------------------------------------------------------------------
// append: one thread per 16-byte chunk of a new token's head row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void append_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                     const int64_t* __restrict__ slots, char* k_cache, char* v_cache,
                                                     int64_t total, int32_t chunks_per_row, int32_t num_kv_heads,
                                                     int32_t row_bytes, int32_t block_size, int64_t num_slots,
                                                     int32_t nhd) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int32_t c = static_cast<int32_t>(idx % chunks_per_row);
  const int64_t rest = idx / chunks_per_row;
  const int32_t jh = static_cast<int32_t>(rest % num_kv_heads);
  const int64_t i = rest / num_kv_heads;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t pb = slot / block_size;
  const int64_t off = slot - pb * block_size;
  const size_t src = (static_cast<size_t>(i) * num_kv_heads + jh) * row_bytes + static_cast<size_t>(c) * 16;
  const size_t row = nhd ? (static_cast<size_t>(pb) * block_size + off) * num_kv_heads + jh
                         : (static_cast<size_t>(pb) * num_kv_heads + jh) * block_size + off;
  const size_t dst = row * row_bytes + static_cast<size_t>(c) * 16;
  const char* s = blockIdx.y ? v : k;
  char* d = blockIdx.y ? v_cache : k_cache;
  *reinterpret_cast<u32x4*>(d + dst) = *reinterpret_cast<const u32x4*>(s + src);
}

// ---------------------------------------------------------------------------
// FP8 append: one wave per (token, KV head, K or V) quantizes the row (scale =
// row amax / 448) and writes codes and scale into the slot
// ---------------------------------------------------------------------------
template <typename Tin, int D, int kQ>
__global__ __launch_bounds__(64) void append_q8_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                        const int64_t* __restrict__ slots, char* k_cache,
                                                        char* v_cache, float* k_scales, float* v_scales,
                                                        int32_t num_kv_heads, int32_t block_size, int64_t num_slots,
                                                        int32_t nhd) {
  constexpr int kPer = D / 64;  // elements per lane
  const int lane = threadIdx.x;
  const int j = blockIdx.x;
  const int64_t i = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  const char* src = (is_v ? v : k) + (i * num_kv_heads + j) * D * static_cast<int64_t>(sizeof(Tin));
  float x[kPer];
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    x[e] = elt_to_float<Tin>(src + (lane * kPer + e) * sizeof(Tin));
    am = fmax_nan(am, fabsf(x[e]));
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) am = fmax_nan(am, xor_shuffle(am, m));
  const RowQuant rq = row_quant<kQ>(am);
  const int64_t pb = slot / block_size;
  const int64_t off = slot - pb * block_size;
  const int64_t row = nhd ? (pb * block_size + off) * num_kv_heads + j : (pb * num_kv_heads + j) * block_size + off;
  char* dst = (is_v ? v_cache : k_cache) + row * D + lane * kPer;
  const unsigned codes = quant4<kQ>(x[0], kPer > 1 ? x[kPer - 1] : 0.f, 0.f, 0.f, rq);
  if constexpr (kPer == 2) *reinterpret_cast<unsigned short*>(dst) = static_cast<unsigned short>(codes & 0xffffu);
  else *reinterpret_cast<unsigned char*>(dst) = static_cast<unsigned char>(codes & 0xffu);
  if (lane == 0) (is_v ? v_scales : k_scales)[row] = rq.scale;
}

// ---------------------------------------------------------------------------
// host-side helpers
// ---------------------------------------------------------------------------
int elt_bytes(pkv_dtype dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
  }
  return 0;
}

int64_t ceil_div64(int64_t x, int64_t y) { return (x + y - 1) / y; }

int32_t auto_partition_tiles_for_units(int64_t units, int64_t max_tiles, int32_t longest = 64) {
  if (units <= 0 || max_tiles <= 0) return 16;
  // Long partitions amortise each workgroup's start-up (table and Q loads,
  // then the first dependent K/V loads) and the merge (one wave combines all
  // of a unit's partitions, four at a time); the halving from `longest` stops
  // once there are PKV_PARTITION_TARGET workgroups (two per CU at the default).
  const int64_t target = PKV_PARTITION_TARGET;
  int32_t pb = longest;
  while (pb > 8 && units * ceil_div64(max_tiles, pb) < target) pb /= 2;
  return pb;
}

int32_t auto_partition_tiles(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int64_t max_tiles) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_heads <= 0) return 16;
  const int64_t group = num_heads / num_kv_heads;
  return auto_partition_tiles_for_units(static_cast<int64_t>(num_seqs) * num_kv_heads * ceil_div64(group, 16),
                                        max_tiles);
}

bool valid_block_size(int32_t block_size) {
  return block_size >= kTile && block_size % kTile == 0 && block_size / kTile <= kMaxPartitionBlocks;
}

// Partition size in cache blocks: `requested` if > 0, else the library's
// choice (a tile count converted to whole blocks). Callers check the block size.
int32_t partition_blocks_for(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t max_blocks,
                             int32_t block_size, int32_t requested) {
  if (requested > 0) return requested;
  const int32_t m = block_size / kTile;
  const int32_t tiles =
      auto_partition_tiles(num_seqs, num_heads, num_kv_heads, static_cast<int64_t>(max_blocks) * m);
  return tiles / m > 0 ? tiles / m : 1;
}

enum Phase : unsigned { kPartitions = 1u, kMerge = 2u, kFusedStep = 4u };

// Compute units of the current device (queried once per device).
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}
// HND fused step: waves per workgroup when the waves are consecutive
// partitions of one unit (sequence, KV head, head group), or 1 to keep the
// head-grouped mapping. `resident(w)` is the number of workgroups of w waves
// one compute unit holds; every choice leaves a workgroup for every compute
// unit. Wide groups leave fewer partials to merge through global memory, and
// a unit that one group covers merges in LDS alone. But a group's last wave
// does that global merge after its siblings have left, and a new workgroup
// needs as many free wave slots on one compute unit as it has waves: in a
// grid that runs in several waves of workgroups, wide groups whose members
// end at different times (ragged batches) leave slots idle. Hence the widest
// groups when the grid is resident all at once or one group covers a unit,
// else groups of 2.
template <typename Resident>
int partition_waves(int64_t parts, int64_t units, Resident resident) {
  if (!PKV_WG_PARTS) return 1;
  const int64_t cus = device_cus();
  for (int w = PKV_DECODE_WAVES; w > 1; w /= 2) {
    const int64_t groups = ceil_div64(parts, w), wgs = groups * units;
    if (parts < w || wgs < cus) continue;
    if (w == 2 || groups == 1 || wgs <= static_cast<int64_t>(resident(w)) * cus) return w;
  }
  return 1;
}
// NHD decode: waves per workgroup, one per KV head: the most (up to
// PKV_DECODE_WAVES, dividing the KV head count) that still leave a workgroup
// for every compute unit.
int decode_waves(int64_t waves, int32_t num_kv_heads) {
  for (int w = PKV_DECODE_WAVES; w > 1; w /= 2)
    if (num_kv_heads % w == 0 && waves / w >= device_cus()) return w;
  return 1;
}

template <typename T, int D, int kQ, bool kNHD>
pkv_status launch_decode(const DecodeArgs& a, int32_t num_seqs, unsigned phases, hipStream_t stream) {
  static_assert(kDecodeWaves<kModeSplit> == kDecodeWaves<kModeStep>, "one bound for both modes");
  // dynamic LDS of the per-wave K ring (8-bit caches of head size 128, HND)
  constexpr bool kRingLds = kQ != 0 && !kNHD && D == 128 && PKV_KRING_8BIT && PKV_DECODE_PAIRS;
  auto ring_bytes = [](int waves) { return kRingLds ? static_cast<size_t>(waves) * kKRingWaveBytes : size_t(0); };
  // waves = consecutive KV heads of one partition
  const int w = decode_waves(static_cast<int64_t>(a.num_parts) * a.num_kv_heads * a.head_groups * num_seqs,
                             a.num_kv_heads);
  const dim3 grid(a.num_parts, static_cast<unsigned>(a.num_kv_heads / w * a.head_groups), num_seqs);
  if (phases & kFusedStep) {
    if constexpr (!kNHD) {  // waves = consecutive partitions of one unit, merged in LDS
      constexpr auto kernel = decode_partition_kernel<T, D, kModeStep, kQ, false, true>;
      // resident workgroups per compute unit, by waves per workgroup (same on every device)
      static const std::array<int, PKV_DECODE_WAVES + 1> occ = [] {
        std::array<int, PKV_DECODE_WAVES + 1> r{};
        for (int v = 2; v <= PKV_DECODE_WAVES; v *= 2) {
          int nb = 0;
          const size_t lds = wg_merge_lds_bytes(v, D) + (kRingLds ? static_cast<size_t>(v) * kKRingWaveBytes : 0);
          if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, 64 * v, lds) != hipSuccess)
            nb = 0;  // unknown: the grouped mapping is not used
          r[v] = nb;
        }
        return r;
      }();
      const int wp = partition_waves(a.num_parts, static_cast<int64_t>(num_seqs) * a.num_kv_heads * a.head_groups,
                                     [&](int v) { return occ[v]; });
      if (wp > 1) {
        // 8-bit codes, grouped-query attention: head pairs share their scale
        // lines through one L2 (E4M3 and INT8 70B step: +1.7% and +2.0%;
        // with one query head per KV head it measured 1.7% slower)
        DecodeArgs g2 = a;
        g2.pair_heads = kQ != 0 && PKV_PAIR_HEADS && a.num_kv_heads % 2 == 0 && a.group > 1;
        const dim3 g(static_cast<unsigned>(ceil_div64(a.num_parts, wp)),
                     static_cast<unsigned>(a.num_kv_heads * a.head_groups), num_seqs);
        hipLaunchKernelGGL(kernel, g, dim3(64 * wp), wg_merge_lds_bytes(wp, D) + ring_bytes(wp), stream, g2);
        return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
      }
    }
    hipLaunchKernelGGL((decode_partition_kernel<T, D, kModeStep, kQ, kNHD>), grid, dim3(64 * w), ring_bytes(w), stream,
                       a);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
  }
  if (phases & kPartitions)
    hipLaunchKernelGGL((decode_partition_kernel<T, D, kModeSplit, kQ, kNHD>), grid, dim3(64 * w), ring_bytes(w),
                       stream, a);
  if ((phases & kMerge) && a.num_parts > 1) {
    const int64_t waves = static_cast<int64_t>(num_seqs) * a.num_heads;
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3(static_cast<unsigned>(ceil_div64(waves, 4))), dim3(256), 0, stream,
                       a, num_seqs);
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

template <typename T, int D, int kQ = 0>
pkv_status launch_layout(const DecodeArgs& a, int32_t num_seqs, unsigned phases, hipStream_t stream, bool nhd) {
  return nhd ? launch_decode<T, D, kQ, true>(a, num_seqs, phases, stream)
             : launch_decode<T, D, kQ, false>(a, num_seqs, phases, stream);
}

template <typename T, int D, int kQ = 0>
pkv_status launch_prefill(const DecodeArgs& a, int32_t num_seqs, hipStream_t stream, bool nhd) {
  dim3 grid(a.num_parts, a.num_kv_heads * a.q_tiles, num_seqs);
  if (nhd) hipLaunchKernelGGL((decode_partition_kernel<T, D, kModePrefill, kQ, true>), grid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL((decode_partition_kernel<T, D, kModePrefill, kQ, false>), grid, dim3(64), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

template <typename T, int D, int kQ = 0>
pkv_status launch_prefill_lds(const DecodeArgs& a, int32_t num_seqs, hipStream_t stream, bool nhd) {
  dim3 grid(a.num_parts, a.num_kv_heads * a.q_tiles, num_seqs);
  constexpr int kW = prefill_waves(D), kR = PKV_PREFILL_LDS_ROWS, kT = PKV_PREFILL_TILES;
  if (nhd) hipLaunchKernelGGL((prefill_lds_kernel<T, D, true, kW, kR, kT, kQ>), grid, dim3(64 * kW), 0, stream, a);
  else hipLaunchKernelGGL((prefill_lds_kernel<T, D, false, kW, kR, kT, kQ>), grid, dim3(64 * kW), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

// 16-bit query type x head size x code format (kQFp8 / kQInt8) for 8-bit caches
template <template <typename, int, int> class L, typename... A>
pkv_status dispatch_codes(pkv_dtype dtype, int head_dim, int q, A&&... args) {
  if (dtype == PKV_BF16) {
    if (q == kQInt8)
      return head_dim == 128 ? L<__bf16, 128, kQInt8>::go(args...) : L<__bf16, 64, kQInt8>::go(args...);
    return head_dim == 128 ? L<__bf16, 128, kQFp8>::go(args...) : L<__bf16, 64, kQFp8>::go(args...);
  }
  if (q == kQInt8)
    return head_dim == 128 ? L<_Float16, 128, kQInt8>::go(args...) : L<_Float16, 64, kQInt8>::go(args...);
  return head_dim == 128 ? L<_Float16, 128, kQFp8>::go(args...) : L<_Float16, 64, kQFp8>::go(args...);
}
template <typename T, int D, int kQ>
struct LayoutLauncher {
  static pkv_status go(const DecodeArgs& a, int32_t num_seqs, unsigned phases, hipStream_t s, bool nhd) {
    return launch_layout<T, D, kQ>(a, num_seqs, phases, s, nhd);
  }
};
template <typename T, int D, int kQ>
struct PrefillLauncher {
  static pkv_status go(const DecodeArgs& a, int32_t num_seqs, hipStream_t s, bool nhd) {
    return launch_prefill<T, D, kQ>(a, num_seqs, s, nhd);
  }
};

size_t workspace_bytes_for(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int64_t parts) {
  if (parts <= 1) return 0;
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_heads * parts;
  return static_cast<size_t>(ceil_div64(rows * head_dim * 4, 256) * 256 + ceil_div64(rows * 4, 256) * 256);
}

// The fused step keeps its partials per work unit (sequence, KV head, head
// group, partition) in the lane-major layout of the kernel: 64 lanes x 4*(D/16)
// floats, then 16 lse values per unit, then one arrival counter per
// (sequence, KV head, head group).
struct StepLayout {
  size_t o_bytes, lse_bytes, ctr_bytes;
  size_t total() const { return o_bytes + lse_bytes + ctr_bytes; }
};
StepLayout merge_layout(int64_t units, int32_t head_dim, int64_t parts) {
  if (parts <= 1) return {0, 0, 0};
  return {static_cast<size_t>(ceil_div64(units * parts * 64 * (head_dim / 4) * 4, 256) * 256),
          static_cast<size_t>(ceil_div64(units * parts * 16 * 4, 256) * 256),
          static_cast<size_t>(ceil_div64(units * 4, 256) * 256)};
}
StepLayout step_layout(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int64_t parts) {
  const int64_t groups = ceil_div64(num_heads / num_kv_heads, 16);
  return merge_layout(static_cast<int64_t>(num_seqs) * num_kv_heads * groups, head_dim, parts);
}
// How a prefill launch splits its rows. The LDS kernel serves 16-bit caches,
// 8-bit caches of head size 128, and positive finite scales: a work unit is a
// workgroup of prefill_waves(head_dim) waves with PKV_PREFILL_LDS_ROWS row
// groups each. fp32 caches, 8-bit caches of head size 64 (and other scales)
// take the one-wave tile kernel with prefill_row_groups(dtype) row groups per unit.
struct PrefillPlan {
  bool lds;
  int32_t rows_per_unit;   // (token, head) rows of one KV head per work unit
  int32_t slots_per_unit;  // 16-row groups per unit: partial slots and counters
  int32_t longest;         // longest automatic partition, 16-row tiles
  int32_t max_tiles;       // longest partition the kernel takes, 16-row tiles
};
PrefillPlan prefill_plan(pkv_dtype dtype, int codes, int32_t head_dim, float scale) {
  const float c = scale * kLog2e;  // the LDS kernel applies c > 0 inside the exponent
  if (PKV_PREFILL_LDS && (codes == 0 || head_dim == 128) && dtype != PKV_F32 && c > 0.f && c <= 3.0e38f) {
    const int32_t groups = prefill_waves(head_dim) * PKV_PREFILL_LDS_ROWS;
    return {true, groups * kTile, groups, kMaxPrefillTiles, kMaxPrefillTiles};
  }
  const int32_t kR = prefill_row_groups(dtype);
  return {false, kR * kTile, kR, 64, kMaxPartitionBlocks};
}
// query tiles (work units) per (sequence, KV head) for a chunk of up to
// max_q_len tokens
int64_t prefill_q_tiles(int32_t num_heads, int32_t num_kv_heads, int32_t max_q_len, const PrefillPlan& plan) {
  return ceil_div64(static_cast<int64_t>(max_q_len) * (num_heads / num_kv_heads), plan.rows_per_unit);
}
// partition size in cache blocks (`requested` if > 0) and the workspace a
// launch with this plan needs
struct PrefillSplit {
  int64_t q_tiles, units;
  int32_t pb, parts;
  size_t ws_bytes;
};
PrefillSplit prefill_split(const PrefillPlan& plan, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t max_q_len, int32_t max_blocks, int32_t block_size,
                           int32_t requested) {
  PrefillSplit r{};
  r.q_tiles = prefill_q_tiles(num_heads, num_kv_heads, max_q_len, plan);
  r.units = static_cast<int64_t>(num_seqs) * num_kv_heads * r.q_tiles;
  const int32_t m = block_size / kTile;
  r.pb = requested;
  if (r.pb <= 0) {
    const int32_t tiles = auto_partition_tiles_for_units(r.units, static_cast<int64_t>(max_blocks) * m, plan.longest);
    r.pb = tiles / m > 0 ? tiles / m : 1;
  }
  r.parts = static_cast<int32_t>(ceil_div64(max_blocks, r.pb));
  r.ws_bytes = merge_layout(r.units * plan.slots_per_unit, head_dim, r.parts).total();
  return r;
}

}  // namespace

// ---------------------------------------------------------------------------
// Library-owned scratch of pkv_decode_step_noalloc (for callers that cannot
// allocate): one fixed array per device, held until the process ends. Its
// first kScratchCounterBytes hold the fused step's arrival counters, the rest
// its partition results. Host code never uses the array's name as an
// address (on the host it only names the symbol): the device address comes
// from hipGetSymbolAddress, once per device, and is kept per device.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(64) << 20;         // 64 MiB in all
constexpr size_t kScratchCounterBytes = size_t(64) << 10;  // 16384 arrival counters
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

// Device address of this device's scratch, set up on its first use: the
// symbol's address with this device current, and its counter region cleared
// by a fill kernel on `stream` (a kernel rather than a memset node, so a
// first call made under graph capture stays correct on every replay).
std::mutex g_scratch_mu;
char* g_scratch_ptr[64] = {};
pkv_status scratch_on_device(hipStream_t stream, char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return PKV_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return PKV_EHIP;
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream, static_cast<uint32_t*>(ptr),
                       static_cast<int64_t>(kScratchCounterBytes / 4));
    if (hipGetLastError() != hipSuccess) return PKV_EHIP;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

// Validate, fill DecodeArgs and launch the requested phases. Pointers the
// chosen phases never read may be null (the merge needs no q or caches).
pkv_status decode_entry(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                        int32_t num_blocks, float scale, void* out, pkv_dtype dtype, const void* workspace,
                        size_t workspace_bytes, int32_t partition_blocks, unsigned phases, void* stream,
                        const void* k_new = nullptr,
                        const void* v_new = nullptr, const float* k_scales = nullptr,
                        const float* v_scales = nullptr, int codes = 0, bool static_scratch = false) {
  const bool fp8 = codes != 0;  // 8-bit codes (E4M3 or INT8) with per-row scales
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0) return PKV_EINVAL;
  if ((phases & kPartitions) && num_blocks <= 0) return PKV_EINVAL;
  if (num_heads % num_kv_heads != 0) return PKV_EINVAL;
  if (elt_bytes(dtype) == 0) return PKV_EINVAL;
  if (!valid_block_size(block_size) || (head_dim != 64 && head_dim != 128)) return PKV_EUNSUPPORTED;
  if (layout != PKV_HND && layout != PKV_NHD) return PKV_EINVAL;
  if (partition_blocks < 0 || static_cast<int64_t>(partition_blocks) * (block_size / kTile) > kMaxPartitionBlocks)
    return PKV_EINVAL;
  // tile addresses are cache row indices and lengths are int32
  if ((phases & (kPartitions | kFusedStep)) &&
      static_cast<int64_t>(num_blocks) * num_kv_heads * block_size > INT32_MAX)
    return PKV_EUNSUPPORTED;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!context_lens || !out) return PKV_EINVAL;
  if ((phases & (kPartitions | kFusedStep)) && (!q || !k_cache || !v_cache || !block_tables)) return PKV_EINVAL;
  if ((phases & kFusedStep) && (!k_new || !v_new)) return PKV_EINVAL;
  if (fp8 && (phases & (kPartitions | kFusedStep)) && (!k_scales || !v_scales)) return PKV_EINVAL;
  if (fp8 && dtype == PKV_F32) return PKV_EUNSUPPORTED;
  if (max_blocks_per_seq == 0) max_blocks_per_seq = 1;  // every length clamps to 0 -> zero rows

  DecodeArgs a{};
  a.q = static_cast<const char*>(q);
  a.k_cache = static_cast<const char*>(k_cache);
  a.v_cache = static_cast<const char*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = static_cast<char*>(out);
  a.max_blocks = max_blocks_per_seq;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.head_groups = (a.group + 15) / 16;
  a.num_blocks = num_blocks;
  const int32_t pb = partition_blocks_for(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq, block_size,
                                          partition_blocks);
  a.tiles_per_block = block_size / kTile;
  a.pb_per_part = pb * a.tiles_per_block;
  a.num_parts = static_cast<int32_t>(ceil_div64(max_blocks_per_seq, pb));
  a.cap_tokens = max_blocks_per_seq * block_size;
  a.qk_scale = scale * kLog2e;
  if (static_cast<int64_t>(num_kv_heads) * a.head_groups > 65535 || num_seqs > 65535) return PKV_EINVAL;
  a.k_scales = reinterpret_cast<const char*>(k_scales);
  a.v_scales = reinterpret_cast<const char*>(v_scales);
  a.k_new = static_cast<const char*>(k_new);
  a.v_new = static_cast<const char*>(v_new);
  a.k_cache_w = const_cast<char*>(static_cast<const char*>(k_cache));
  a.v_cache_w = const_cast<char*>(static_cast<const char*>(v_cache));
  if (a.num_parts > 1) {
    char* ws = const_cast<char*>(static_cast<const char*>(workspace));
    if ((phases & kFusedStep) && static_scratch) {
      // the library's own device array: counters at its start (a fixed place,
      // so every completed call leaves them zero for the next, whatever its
      // shape), then partials and lse values
      const StepLayout L = step_layout(num_seqs, num_heads, num_kv_heads, head_dim, a.num_parts);
      if (L.ctr_bytes > kScratchCounterBytes || L.o_bytes + L.lse_bytes > kScratchBytes - kScratchCounterBytes)
        return PKV_ESMALL;
      char* sp = nullptr;
      const pkv_status st = scratch_on_device(static_cast<hipStream_t>(stream), &sp);
      if (st != PKV_OK) return st;
      a.counters = reinterpret_cast<int32_t*>(sp);
      a.ws_o = reinterpret_cast<float*>(sp + kScratchCounterBytes);
      a.ws_lse = reinterpret_cast<float*>(sp + kScratchCounterBytes + L.o_bytes);
    } else if (phases & kFusedStep) {
      const StepLayout L = step_layout(num_seqs, num_heads, num_kv_heads, head_dim, a.num_parts);
      if (!workspace || workspace_bytes < L.total()) return PKV_ESMALL;
      a.ws_o = reinterpret_cast<float*>(ws);
      a.ws_lse = reinterpret_cast<float*>(ws + L.o_bytes);
      a.counters = reinterpret_cast<int32_t*>(ws + L.o_bytes + L.lse_bytes);
    } else {
      const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, a.num_parts);
      if (!workspace || workspace_bytes < need) return PKV_ESMALL;
      const int64_t rows = static_cast<int64_t>(num_seqs) * num_heads * a.num_parts;
      a.ws_o = reinterpret_cast<float*>(ws);
      a.ws_lse = reinterpret_cast<float*>(ws + ceil_div64(rows * head_dim * 4, 256) * 256);
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool nhd = layout == PKV_NHD;
  if (fp8) return dispatch_codes<LayoutLauncher>(dtype, head_dim, codes, a, num_seqs, phases, s, nhd);
  switch (dtype) {
    case PKV_BF16:
      return head_dim == 128 ? launch_layout<__bf16, 128>(a, num_seqs, phases, s, nhd)
                             : launch_layout<__bf16, 64>(a, num_seqs, phases, s, nhd);
    case PKV_F16:
      return head_dim == 128 ? launch_layout<_Float16, 128>(a, num_seqs, phases, s, nhd)
                             : launch_layout<_Float16, 64>(a, num_seqs, phases, s, nhd);
    case PKV_F32:
      return head_dim == 128 ? launch_layout<float, 128>(a, num_seqs, phases, s, nhd)
                             : launch_layout<float, 64>(a, num_seqs, phases, s, nhd);
  }
  return PKV_EINVAL;
}

// Chunked prefill: validate, fill DecodeArgs for kModePrefill and launch.
pkv_status prefill_entry(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* q_start, int32_t max_q_len,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, pkv_layout layout, int32_t num_blocks, float scale,
                         void* out, pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                         int32_t partition_blocks, void* stream, const float* k_scales, const float* v_scales,
                         int codes) {
  const bool fp8 = codes != 0;  // 8-bit codes (E4M3 or INT8) with per-row scales
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0 || max_q_len < 0)
    return PKV_EINVAL;
  if (num_blocks <= 0 || num_heads % num_kv_heads != 0 || elt_bytes(dtype) == 0) return PKV_EINVAL;
  if (!valid_block_size(block_size) || (head_dim != 64 && head_dim != 128)) return PKV_EUNSUPPORTED;
  if (layout != PKV_HND && layout != PKV_NHD) return PKV_EINVAL;
  const PrefillPlan plan = prefill_plan(dtype, codes, head_dim, scale);
  if (partition_blocks < 0 || static_cast<int64_t>(partition_blocks) * (block_size / kTile) > plan.max_tiles)
    return PKV_EINVAL;
  if (static_cast<int64_t>(num_blocks) * num_kv_heads * block_size > INT32_MAX) return PKV_EUNSUPPORTED;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX) return PKV_EINVAL;
  if (fp8 && dtype == PKV_F32) return PKV_EUNSUPPORTED;
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !q_start || !context_lens || !out) return PKV_EINVAL;
  if (fp8 && (!k_scales || !v_scales)) return PKV_EINVAL;
  if (max_blocks_per_seq == 0) max_blocks_per_seq = 1;
  const PrefillSplit split = prefill_split(plan, num_seqs, num_heads, num_kv_heads, head_dim, max_q_len,
                                           max_blocks_per_seq, block_size, partition_blocks);
  const int64_t qt = split.q_tiles;
  if (qt * num_kv_heads > 65535 || num_seqs > 65535) return PKV_EINVAL;
  DecodeArgs a{};
  a.q = static_cast<const char*>(q);
  a.k_cache = static_cast<const char*>(k_cache);
  a.v_cache = static_cast<const char*>(v_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = static_cast<char*>(out);
  a.max_blocks = max_blocks_per_seq;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.head_groups = 1;
  a.num_blocks = num_blocks;
  a.q_start = q_start;
  a.max_q_len = max_q_len;
  a.q_tiles = static_cast<int32_t>(qt);
  const int32_t m = block_size / kTile;
  a.tiles_per_block = m;
  a.pb_per_part = split.pb * m;
  a.num_parts = split.parts;
  a.cap_tokens = max_blocks_per_seq * block_size;
  a.qk_scale = scale * kLog2e;
  a.k_scales = reinterpret_cast<const char*>(k_scales);
  a.v_scales = reinterpret_cast<const char*>(v_scales);
  if (a.num_parts > 1) {
    const StepLayout L = merge_layout(split.units * plan.slots_per_unit, head_dim, a.num_parts);  // slot per row group
    if (!workspace || workspace_bytes < L.total()) return PKV_ESMALL;
    char* ws = static_cast<char*>(workspace);
    a.ws_o = reinterpret_cast<float*>(ws);
    a.ws_lse = reinterpret_cast<float*>(ws + L.o_bytes);
    a.counters = reinterpret_cast<int32_t*>(ws + L.o_bytes + L.lse_bytes);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool nhd = layout == PKV_NHD;
  if (fp8 && plan.lds) {  // head size 128
    const bool i8 = codes == kQInt8;
    if (dtype == PKV_BF16)
      return i8 ? launch_prefill_lds<__bf16, 128, kQInt8>(a, num_seqs, s, nhd)
                : launch_prefill_lds<__bf16, 128, kQFp8>(a, num_seqs, s, nhd);
    return i8 ? launch_prefill_lds<_Float16, 128, kQInt8>(a, num_seqs, s, nhd)
              : launch_prefill_lds<_Float16, 128, kQFp8>(a, num_seqs, s, nhd);
  }
  if (fp8) return dispatch_codes<PrefillLauncher>(dtype, head_dim, codes, a, num_seqs, s, nhd);
  if (plan.lds) {
    if (dtype == PKV_BF16)
      return head_dim == 128 ? launch_prefill_lds<__bf16, 128>(a, num_seqs, s, nhd)
                             : launch_prefill_lds<__bf16, 64>(a, num_seqs, s, nhd);
    return head_dim == 128 ? launch_prefill_lds<_Float16, 128>(a, num_seqs, s, nhd)
                           : launch_prefill_lds<_Float16, 64>(a, num_seqs, s, nhd);
  }
  switch (dtype) {
    case PKV_BF16:
      return head_dim == 128 ? launch_prefill<__bf16, 128>(a, num_seqs, s, nhd)
                             : launch_prefill<__bf16, 64>(a, num_seqs, s, nhd);
    case PKV_F16:
      return head_dim == 128 ? launch_prefill<_Float16, 128>(a, num_seqs, s, nhd)
                             : launch_prefill<_Float16, 64>(a, num_seqs, s, nhd);
    case PKV_F32:
      return head_dim == 128 ? launch_prefill<float, 128>(a, num_seqs, s, nhd)
                             : launch_prefill<float, 64>(a, num_seqs, s, nhd);
  }
  return PKV_EINVAL;
}

// quantizing append of either code format
template <int kQ>
pkv_status append_codes(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                        void* k_cache, void* v_cache, float* k_scales, float* v_scales, int32_t num_blocks,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                        pkv_dtype dtype, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0) return PKV_EINVAL;
  if (layout != PKV_HND && layout != PKV_NHD) return PKV_EINVAL;
  if (elt_bytes(dtype) == 0) return PKV_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if (num_kv_heads > 65535 || num_tokens > 65535) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_scales || !v_scales) return PKV_EINVAL;
  dim3 grid(num_kv_heads, num_tokens, 2);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(64), 0, s, static_cast<const char*>(k), static_cast<const char*>(v),
                       slot_mapping, static_cast<char*>(k_cache), static_cast<char*>(v_cache), k_scales, v_scales,
                       num_kv_heads, block_size, num_slots, static_cast<int32_t>(layout == PKV_NHD));
  };
  switch (dtype) {
    case PKV_F32:
      head_dim == 128 ? go(append_q8_kernel<float, 128, kQ>) : go(append_q8_kernel<float, 64, kQ>);
      break;
    case PKV_F16:
      head_dim == 128 ? go(append_q8_kernel<_Float16, 128, kQ>) : go(append_q8_kernel<_Float16, 64, kQ>);
      break;
    case PKV_BF16:
      head_dim == 128 ? go(append_q8_kernel<__bf16, 128, kQ>) : go(append_q8_kernel<__bf16, 64, kQ>);
      break;
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

template <int NC>
pkv_status launch_stream(const StreamArgs& a, int32_t num_seqs, bool scales, hipStream_t stream) {
  const int w = decode_waves(static_cast<int64_t>(a.num_parts) * a.num_kv_heads * num_seqs, a.num_kv_heads);
  const dim3 grid(a.num_parts, static_cast<unsigned>(a.num_kv_heads / w), num_seqs);
  if (scales) hipLaunchKernelGGL((stream_tiles_kernel<NC, true>), grid, dim3(64 * w), 0, stream, a);
  else hipLaunchKernelGGL((stream_tiles_kernel<NC, false>), grid, dim3(64 * w), 0, stream, a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // namespace

extern "C" {

const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "PKV_OK";
    case PKV_EINVAL: return "PKV_EINVAL: invalid argument";
    case PKV_ERANGE: return "PKV_ERANGE: value out of range";
    case PKV_ENOMEM: return "PKV_ENOMEM: block pool exhausted";
    case PKV_EBUSY: return "PKV_EBUSY: shared block or duplicate slot";
    case PKV_EUNSUPPORTED: return "PKV_EUNSUPPORTED: shape not supported";
    case PKV_EHIP: return "PKV_EHIP: HIP runtime error";
    case PKV_ESMALL: return "PKV_ESMALL: buffer too small";
  }
  return "PKV_?: unknown status";
}

int32_t pkv_version(void) { return 200; }

pkv_status pkv_kv_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                         void* k_cache, void* v_cache, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, pkv_layout layout, pkv_dtype dtype, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return PKV_EINVAL;
  if (layout != PKV_HND && layout != PKV_NHD) return PKV_EINVAL;
  const int eb = elt_bytes(dtype);
  if (eb == 0) return PKV_EINVAL;
  if ((head_dim * eb) % 16 != 0) return PKV_EUNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PKV_EINVAL;
  const int32_t row_bytes = head_dim * eb;
  const int32_t chunks = row_bytes / 16;
  const int64_t total = static_cast<int64_t>(num_tokens) * num_kv_heads * chunks;
  const int64_t blocks = ceil_div64(total, 256);
  if (blocks > 0x7fffffff) return PKV_EINVAL;
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<unsigned>(blocks), 2), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(k), static_cast<const char*>(v),
                     slot_mapping, static_cast<char*>(k_cache), static_cast<char*>(v_cache), total, chunks,
                     num_kv_heads, row_bytes, block_size, static_cast<int64_t>(num_blocks) * block_size,
                     static_cast<int32_t>(layout == PKV_NHD));
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

int32_t pkv_decode_partition_blocks(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t max_blocks_per_seq, int32_t block_size) {
  if (!valid_block_size(block_size)) return 0;
  return partition_blocks_for(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq, block_size, 0);
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_blocks) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0) return 0;
  if (!valid_block_size(block_size)) return 0;
  const int32_t pb = partition_blocks_for(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq, block_size,
                                          partition_blocks);
  return workspace_bytes_for(num_seqs, num_heads, head_dim, ceil_div64(max_blocks_per_seq, pb));
}

pkv_status pkv_paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                                      int32_t num_blocks, float scale, void* out, pkv_dtype dtype, void* workspace,
                                      size_t workspace_bytes, int32_t partition_blocks, void* stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype, workspace,
                      workspace_bytes, partition_blocks, kPartitions | kMerge, stream);
}

pkv_status pkv_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, pkv_layout layout, int32_t num_blocks, float scale, void* out,
                                 pkv_dtype dtype, void* workspace, size_t workspace_bytes, int32_t partition_blocks,
                                 void* stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype, workspace,
                      workspace_bytes, partition_blocks, kPartitions, stream);
}

size_t pkv_decode_step_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_blocks) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0) return 0;
  if (!valid_block_size(block_size)) return 0;
  const int32_t pb = partition_blocks_for(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq, block_size,
                                          partition_blocks);
  return step_layout(num_seqs, num_heads, num_kv_heads, head_dim, ceil_div64(max_blocks_per_seq, pb)).total();
}

pkv_status pkv_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, pkv_layout layout, int32_t num_blocks, float scale, void* out,
                           pkv_dtype dtype, void* workspace, size_t workspace_bytes, int32_t partition_blocks,
                           void* stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype, workspace,
                      workspace_bytes, partition_blocks, kFusedStep, stream, k_new, v_new);
}

pkv_status pkv_decode_step_noalloc(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                   void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                                   int32_t num_blocks, float scale, void* out, pkv_dtype dtype,
                                   int32_t partition_blocks, void* stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype, nullptr, 0,
                      partition_blocks, kFusedStep, stream, k_new, v_new, nullptr, nullptr, 0, true);
}

pkv_status pkv_copy_blocks(void* const* caches, const int64_t* block_bytes, int32_t n_caches, int32_t num_blocks,
                           const int32_t* pairs, int32_t n_pairs, void* stream) {
  if (n_caches < 1 || n_caches > 4 || num_blocks <= 0 || n_pairs < 0 || !caches || !block_bytes) return PKV_EINVAL;
  CopyArgs a{};
  for (int c = 0; c < n_caches; ++c) {
    if (!caches[c] || reinterpret_cast<uintptr_t>(caches[c]) % 16 != 0) return PKV_EINVAL;
    if (block_bytes[c] <= 0 || block_bytes[c] % 16 != 0) return PKV_EINVAL;
    if (block_bytes[c] > INT64_MAX / num_blocks) return PKV_EINVAL;
    a.base[c] = static_cast<char*>(caches[c]);
    a.bytes[c] = block_bytes[c];
  }
  if (n_pairs == 0) return PKV_OK;
  if (!pairs) return PKV_EINVAL;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n_pairs, n_caches), dim3(256), 0, static_cast<hipStream_t>(stream), a,
                     pairs, num_blocks);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

pkv_status pkv_kv_append_fp8(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                             void* k_cache, void* v_cache, float* k_scales, float* v_scales, int32_t num_blocks,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                             pkv_dtype dtype, void* stream) {
  return append_codes<kQFp8>(k, v, slot_mapping, num_tokens, k_cache, v_cache, k_scales, v_scales, num_blocks,
                             num_kv_heads, head_dim, block_size, layout, dtype, stream);
}

pkv_status pkv_kv_append_int8(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                              void* k_cache, void* v_cache, float* k_scales, float* v_scales, int32_t num_blocks,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                              pkv_dtype dtype, void* stream) {
  return append_codes<kQInt8>(k, v, slot_mapping, num_tokens, k_cache, v_cache, k_scales, v_scales, num_blocks,
                              num_kv_heads, head_dim, block_size, layout, dtype, stream);
}

pkv_status pkv_paged_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache,
                                          const float* k_scales, const float* v_scales,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                          pkv_layout layout, int32_t num_blocks, float scale, void* out,
                                          pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                          int32_t partition_blocks, void* stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype, workspace,
                      workspace_bytes, partition_blocks, kPartitions | kMerge, stream, nullptr, nullptr, k_scales,
                      v_scales, kQFp8);
}

pkv_status pkv_decode_step_fp8(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               float* k_scales, float* v_scales, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               pkv_layout layout, int32_t num_blocks, float scale, void* out, pkv_dtype dtype,
                               void* workspace, size_t workspace_bytes, int32_t partition_blocks, void* stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype, workspace,
                      workspace_bytes, partition_blocks, kFusedStep, stream, k_new, v_new, k_scales, v_scales, kQFp8);
}

size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_q_len, int32_t max_blocks_per_seq, int32_t block_size,
                                   int32_t partition_blocks) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_q_len <= 0 ||
      max_blocks_per_seq <= 0 || num_heads % num_kv_heads != 0 || !valid_block_size(block_size))
    return 0;
  // enough for every plan (the launch's dtype, cache format and scale decide which)
  size_t need = 0;
  const PrefillPlan plans[] = {prefill_plan(PKV_BF16, 0, head_dim, 1.f), prefill_plan(PKV_BF16, kQFp8, head_dim, 1.f),
                               prefill_plan(PKV_BF16, 0, head_dim, -1.f), prefill_plan(PKV_F32, 0, head_dim, 1.f)};
  for (const PrefillPlan& plan : plans) {
    const size_t bytes = prefill_split(plan, num_seqs, num_heads, num_kv_heads, head_dim, max_q_len,
                                       max_blocks_per_seq, block_size, partition_blocks).ws_bytes;
    need = bytes > need ? bytes : need;
  }
  return need;
}

pkv_status pkv_prefill_attention(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* q_start,
                                 int32_t max_q_len, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                                 int32_t num_blocks, float scale, void* out, pkv_dtype dtype, void* workspace,
                                 size_t workspace_bytes, int32_t partition_blocks, void* stream) {
  return prefill_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, q_start, max_q_len, context_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype,
                       workspace, workspace_bytes, partition_blocks, stream, nullptr, nullptr, 0);
}

pkv_status pkv_prefill_attention_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scales,
                                     const float* v_scales, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* q_start, int32_t max_q_len, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, pkv_layout layout, int32_t num_blocks, float scale,
                                     void* out, pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                     int32_t partition_blocks, void* stream) {
  return prefill_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, q_start, max_q_len, context_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype,
                       workspace, workspace_bytes, partition_blocks, stream, k_scales, v_scales, kQFp8);
}

pkv_status pkv_paged_decode_attention_int8(const void* q, const void* k_cache, const void* v_cache,
                                           const float* k_scales, const float* v_scales,
                                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                           pkv_layout layout, int32_t num_blocks, float scale, void* out,
                                           pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                           int32_t partition_blocks, void* stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype, workspace,
                      workspace_bytes, partition_blocks, kPartitions | kMerge, stream, nullptr, nullptr, k_scales,
                      v_scales, kQInt8);
}

pkv_status pkv_decode_step_int8(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                float* k_scales, float* v_scales, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                pkv_layout layout, int32_t num_blocks, float scale, void* out, pkv_dtype dtype,
                                void* workspace, size_t workspace_bytes, int32_t partition_blocks, void* stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype, workspace,
                      workspace_bytes, partition_blocks, kFusedStep, stream, k_new, v_new, k_scales, v_scales, kQInt8);
}

pkv_status pkv_prefill_attention_int8(const void* q, const void* k_cache, const void* v_cache, const float* k_scales,
                                      const float* v_scales, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* q_start, int32_t max_q_len, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, pkv_layout layout, int32_t num_blocks, float scale,
                                      void* out, pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                      int32_t partition_blocks, void* stream) {
  return prefill_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, q_start, max_q_len, context_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, layout, num_blocks, scale, out, dtype,
                       workspace, workspace_bytes, partition_blocks, stream, k_scales, v_scales, kQInt8);
}

pkv_status pkv_decode_merge(const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_blocks, void* out,
                            pkv_dtype dtype, void* stream) {
  return decode_entry(nullptr, nullptr, nullptr, nullptr, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, PKV_HND, 1, 0.f, out, dtype, workspace, workspace_bytes,
                      partition_blocks, kMerge, stream);
}

pkv_status pkv_stream_tiles(const void* k_cache, const void* v_cache, const float* k_scales, const float* v_scales,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_kv_heads, int32_t row_bytes, int32_t block_size,
                            pkv_layout layout, int32_t num_blocks, int32_t partition_blocks, uint32_t* sink,
                            size_t sink_words, void* stream) {
  if (num_seqs < 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0 || num_blocks <= 0) return PKV_EINVAL;
  if (layout != PKV_HND && layout != PKV_NHD) return PKV_EINVAL;
  if (row_bytes != 64 && row_bytes != 128 && row_bytes != 256 && row_bytes != 512) return PKV_EUNSUPPORTED;
  if (!valid_block_size(block_size)) return PKV_EUNSUPPORTED;
  if (partition_blocks <= 0 || static_cast<int64_t>(partition_blocks) * (block_size / kTile) > kMaxPartitionBlocks)
    return PKV_EINVAL;
  if ((k_scales == nullptr) != (v_scales == nullptr)) return PKV_EINVAL;
  if (static_cast<int64_t>(num_blocks) * num_kv_heads * block_size > INT32_MAX) return PKV_EUNSUPPORTED;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX) return PKV_EINVAL;
  if (num_kv_heads > 65535 || num_seqs > 65535) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_tables || !context_lens || !sink) return PKV_EINVAL;
  if (max_blocks_per_seq == 0) max_blocks_per_seq = 1;
  StreamArgs a{};
  a.k = static_cast<const char*>(k_cache);
  a.v = static_cast<const char*>(v_cache);
  a.ks = reinterpret_cast<const char*>(k_scales);
  a.vs = reinterpret_cast<const char*>(v_scales);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.sink = sink;
  a.max_blocks = max_blocks_per_seq;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.tiles_per_block = block_size / kTile;
  a.pb_per_part = partition_blocks * a.tiles_per_block;
  a.num_parts = static_cast<int32_t>(ceil_div64(max_blocks_per_seq, partition_blocks));
  a.cap_tokens = max_blocks_per_seq * block_size;
  a.row_bytes = row_bytes;
  a.nhd = layout == PKV_NHD;
  if (sink_words < static_cast<size_t>(num_seqs) * num_kv_heads * a.num_parts * 64) return PKV_ESMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool sc = k_scales != nullptr;
  switch (row_bytes) {
    case 64: return launch_stream<1>(a, num_seqs, sc, s);
    case 128: return launch_stream<2>(a, num_seqs, sc, s);
    case 256: return launch_stream<4>(a, num_seqs, sc, s);
    default: return launch_stream<8>(a, num_seqs, sc, s);
  }
}

}  // extern "C"
