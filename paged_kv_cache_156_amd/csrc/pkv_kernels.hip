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
// Work decomposition (one wavefront = one workgroup):
//   (sequence b, KV head j, head group hg, context partition p).
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
// the maxima shared by the four lanes of a head through two xor-shuffles.
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

namespace {

using f32x4 = float __attribute__((ext_vector_type(4)));
using u32x4 = unsigned __attribute__((ext_vector_type(4)));
using u32x2 = unsigned __attribute__((ext_vector_type(2)));
using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using f16x8 = _Float16 __attribute__((ext_vector_type(8)));
using s16x4 = short __attribute__((ext_vector_type(4)));
using f16x4 = _Float16 __attribute__((ext_vector_type(4)));

constexpr int kBlockSize = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xor_shuffle(float v, int mask) {
  const int lane = static_cast<int>(__lane_id());
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
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

template <int NDW>
__device__ __forceinline__ void load_dwords(unsigned (&dst)[NDW], const char* src) {
  if constexpr (NDW == 2) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(src);
    dst[0] = v[0];
    dst[1] = v[1];
  } else {
    static_assert(NDW % 4 == 0, "row slice must be 8 bytes or a multiple of 16");
#pragma unroll
    for (int w = 0; w < NDW; w += 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + w * 4);
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
  static constexpr int kTileBytes = kBlockSize * kRowBytes;
  static_assert(kRowBytes % 64 == 0, "head row must split into 4 x 16-byte chunk groups");
};

template <typename T, int D>
struct BlockRegs {
  u32x4 k[Shape<T, D>::kNK];
  unsigned v[4][Shape<T, D>::kVDW];
};

template <typename T, int D>
__device__ __forceinline__ void load_block(BlockRegs<T, D>& r, const char* kt, const char* vt, int q4, int ln) {
  using S = Shape<T, D>;
#pragma unroll
  for (int c = 0; c < S::kNK; ++c)
    r.k[c] = *reinterpret_cast<const u32x4*>(kt + ln * S::kRowBytes + (4 * c + q4) * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) load_dwords<S::kVDW>(r.v[i], vt + (4 * q4 + i) * S::kRowBytes + ln * S::kE * S::kElt);
}

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
  int32_t pb_per_part;  // blocks per partition (<= 64)
  int32_t num_parts;    // P
  float qk_scale;       // scale * log2(e)
};

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_partition_kernel(DecodeArgs a) {
  using S = Shape<T, D>;
  constexpr bool k16 = sizeof(T) == 2;
  const int lane = threadIdx.x;
  const int q4 = lane >> 4;
  const int ln = lane & 15;
  const int p = blockIdx.x;
  const int j = blockIdx.y / a.head_groups;
  const int hg = blockIdx.y - j * a.head_groups;
  const int b = blockIdx.z;

  const int cap = a.max_blocks * kBlockSize;
  int n = a.context_lens[b];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int nblk_seq = (n + kBlockSize - 1) / kBlockSize;
  const int nparts = nblk_seq == 0 ? 1 : (nblk_seq + a.pb_per_part - 1) / a.pb_per_part;
  if (p >= nparts) return;
  const int blk0 = p * a.pb_per_part;
  const int nblk = min(a.pb_per_part, nblk_seq - blk0);  // may be 0 only when n == 0

  // this lane's query head (column of the score tile)
  const int hin = hg * 16 + ln;                 // head index inside the GQA group
  const bool head_ok = hin < a.group;
  const int hq = j * a.group + (head_ok ? hin : 0);

  // Q as the B operand, same chunk permutation as K
  u32x4 qv[S::kNK];
  {
    const char* qrow = a.q + (static_cast<size_t>(b) * a.num_heads + hq) * S::kRowBytes;
#pragma unroll
    for (int c = 0; c < S::kNK; ++c)
      qv[c] = head_ok ? *reinterpret_cast<const u32x4*>(qrow + (4 * c + q4) * 16) : u32x4{0, 0, 0, 0};
  }

  // physical ids of this partition's blocks: lane i holds block blk0 + i
  int my_id = 0;
  if (lane < nblk) my_id = a.block_tables[static_cast<size_t>(b) * a.max_blocks + blk0 + lane];

  const size_t head_off = static_cast<size_t>(j) * S::kTileBytes;
  const size_t block_stride = static_cast<size_t>(a.num_kv_heads) * S::kTileBytes;

  f32x4 acc[S::kE];
#pragma unroll
  for (int mt = 0; mt < S::kE; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;  // running max of scaled scores (log2 units)
  float l_run = 0.f;      // this lane's share of the running denominator

  auto block_ptr = [&](int t, bool& ok) -> size_t {
    int id = __builtin_amdgcn_readlane(my_id, t);
    ok = static_cast<unsigned>(id) < static_cast<unsigned>(a.num_blocks);
    return (ok ? static_cast<size_t>(id) : 0) * block_stride + head_off;
  };

  auto process = [&](BlockRegs<T, D>& r, int t, bool ok) {
    const int tok0 = (blk0 + t) * kBlockSize;
    const int valid = ok ? min(kBlockSize, n - tok0) : 0;  // tokens of this block in range
    // scores
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (k16) {
#pragma unroll
      for (int c = 0; c < S::kNK; ++c) s = mfma_qk16<T>(r.k[c], qv[c], s);
    } else {
#pragma unroll
      for (int c = 0; c < S::kNK; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(r.k[c][e]), __uint_as_float(qv[c][e]), s, 0, 0, 0);
    }
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = s[i] * a.qk_scale;
    if (valid < kBlockSize) {  // wave-uniform: only the last block of a sequence, or a bad id
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = 4 * q4 + i < valid;
        sc[i] = in ? sc[i] : kNegInf;
        if (!in) {
#pragma unroll
          for (int w = 0; w < S::kVDW; ++w) r.v[i][w] = 0u;  // select, never multiply, NaN padding
        }
      }
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, xor_shuffle(mx, 16));
    mx = fmaxf(mx, xor_shuffle(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(sc[i] - m_use);
#pragma unroll
    for (int mt = 0; mt < S::kE; ++mt) acc[mt] *= alpha;
    if constexpr (k16) {
      // P^T operand: each weight is split into a 16-bit head plus a 16-bit
      // residual (two MFMAs against the same V tile), so the weights carry
      // about 16 significant bits instead of 8 (bf16) or 11 (fp16)
      unsigned ph[4], pl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ph[i] = to_bits16<T>(pr[i]);
        pl[i] = to_bits16<T>(pr[i] - from_bits16<T>(ph[i]));
      }
      l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      const u32x2 pw_hi = {ph[0] | (ph[1] << 16), ph[2] | (ph[3] << 16)};
      const u32x2 pw_lo = {pl[0] | (pl[1] << 16), pl[2] | (pl[3] << 16)};
#pragma unroll
      for (int mt = 0; mt < S::kE; ++mt) {
        const unsigned sel = (mt & 1) ? 0x07060302u : 0x05040100u;
        const u32x2 av = {__builtin_amdgcn_perm(r.v[1][mt >> 1], r.v[0][mt >> 1], sel),
                          __builtin_amdgcn_perm(r.v[3][mt >> 1], r.v[2][mt >> 1], sel)};
        acc[mt] = mfma_pv16<T>(av, pw_hi, acc[mt]);
        acc[mt] = mfma_pv16<T>(av, pw_lo, acc[mt]);
      }
    } else {
      l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < S::kE; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(r.v[i][mt]), pr[i], acc[mt], 0, 0, 0);
    }
  };

  // stream the partition's blocks, one block of loads in flight ahead
  BlockRegs<T, D> r0, r1;
  bool ok0 = false, ok1 = false;
  if (nblk > 0) {
    const size_t off = block_ptr(0, ok0);
    load_block<T, D>(r0, a.k_cache + off, a.v_cache + off, q4, ln);
  }
  for (int t = 0; t < nblk; t += 2) {
    if (t + 1 < nblk) {
      const size_t off = block_ptr(t + 1, ok1);
      load_block<T, D>(r1, a.k_cache + off, a.v_cache + off, q4, ln);
    }
    process(r0, t, ok0);
    if (t + 1 >= nblk) break;
    if (t + 2 < nblk) {
      const size_t off = block_ptr(t + 2, ok0);
      load_block<T, D>(r0, a.k_cache + off, a.v_cache + off, q4, ln);
    }
    process(r1, t + 1, ok1);
  }

  // combine the four lanes' partial denominators of each head
  float l_tot = l_run + xor_shuffle(l_run, 16);
  l_tot += xor_shuffle(l_tot, 32);
  if (!head_ok) return;
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;

  if (nparts == 1) {
    char* orow = a.out + (static_cast<size_t>(b) * a.num_heads + hq) * S::kRowBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = (4 * q4 + i) * S::kE;
      if constexpr (k16) {
        unsigned w[S::kVDW];
#pragma unroll
        for (int mt = 0; mt < S::kE; mt += 2)
          w[mt >> 1] = to_bits16<T>(acc[mt][i] * inv) | (to_bits16<T>(acc[mt + 1][i] * inv) << 16);
        store_dwords<S::kVDW>(orow + d0 * S::kElt, w);
      } else {
        unsigned w[S::kVDW];
#pragma unroll
        for (int mt = 0; mt < S::kE; ++mt) w[mt] = __float_as_uint(acc[mt][i] * inv);
        store_dwords<S::kVDW>(orow + d0 * S::kElt, w);
      }
    }
  } else {
    const size_t row = (static_cast<size_t>(b) * a.num_heads + hq) * a.num_parts + p;
    float* o = a.ws_o + row * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = (4 * q4 + i) * S::kE;
#pragma unroll
      for (int mt = 0; mt < S::kE; mt += 4)
        *reinterpret_cast<f32x4*>(o + d0 + mt) =
            f32x4{acc[mt][i] * inv, acc[mt + 1][i] * inv, acc[mt + 2][i] * inv, acc[mt + 3][i] * inv};
    }
    if (q4 == 0) a.ws_lse[row] = m_run + __builtin_amdgcn_logf(l_tot);
  }
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
  const int cap = a.max_blocks * kBlockSize;
  int n = a.context_lens[b];
  n = n < 0 ? 0 : (n > cap ? cap : n);
  const int nblk_seq = (n + kBlockSize - 1) / kBlockSize;
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
// append: one thread per 16-byte chunk of a new token's head row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void append_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                     const int64_t* __restrict__ slots, char* k_cache, char* v_cache,
                                                     int64_t total, int32_t chunks_per_row, int32_t num_kv_heads,
                                                     int32_t row_bytes, int32_t block_size, int64_t num_slots) {
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
  const size_t dst = ((static_cast<size_t>(pb) * num_kv_heads + jh) * block_size + off) * row_bytes +
                     static_cast<size_t>(c) * 16;
  const char* s = blockIdx.y ? v : k;
  char* d = blockIdx.y ? v_cache : k_cache;
  *reinterpret_cast<u32x4*>(d + dst) = *reinterpret_cast<const u32x4*>(s + src);
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

int32_t auto_partition_blocks(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t max_blocks) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_heads <= 0 || max_blocks <= 0) return 16;
  const int64_t group = num_heads / num_kv_heads;
  const int64_t units = static_cast<int64_t>(num_seqs) * num_kv_heads * ceil_div64(group, 16);
  // enough single-wave workgroups to keep every CU streaming (256 CUs x 16)
  const int64_t target = 4096;
  int32_t pb = 64;
  while (pb > 8 && units * ceil_div64(max_blocks, pb) < target) pb /= 2;
  return pb;
}

enum Phase : unsigned { kPartitions = 1u, kMerge = 2u };

template <typename T, int D>
pkv_status launch_decode(const DecodeArgs& a, int32_t num_seqs, unsigned phases, hipStream_t stream) {
  if (phases & kPartitions) {
    dim3 grid(a.num_parts, a.num_kv_heads * a.head_groups, num_seqs);
    hipLaunchKernelGGL((decode_partition_kernel<T, D>), grid, dim3(64), 0, stream, a);
  }
  if ((phases & kMerge) && a.num_parts > 1) {
    const int64_t waves = static_cast<int64_t>(num_seqs) * a.num_heads;
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3(static_cast<unsigned>(ceil_div64(waves, 4))), dim3(256), 0, stream,
                       a, num_seqs);
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

size_t workspace_bytes_for(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int64_t parts) {
  if (parts <= 1) return 0;
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_heads * parts;
  return static_cast<size_t>(ceil_div64(rows * head_dim * 4, 256) * 256 + ceil_div64(rows * 4, 256) * 256);
}

// Validate, fill DecodeArgs and launch the requested phases. Pointers the
// chosen phases never read may be null (the merge needs no q or caches).
pkv_status decode_entry(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                        void* out, pkv_dtype dtype, const void* workspace, size_t workspace_bytes,
                        int32_t partition_blocks, unsigned phases, void* stream) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0) return PKV_EINVAL;
  if ((phases & kPartitions) && num_blocks <= 0) return PKV_EINVAL;
  if (num_heads % num_kv_heads != 0) return PKV_EINVAL;
  if (elt_bytes(dtype) == 0) return PKV_EINVAL;
  if (block_size != kBlockSize || (head_dim != 64 && head_dim != 128)) return PKV_EUNSUPPORTED;
  if (partition_blocks < 0 || partition_blocks > 64) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!context_lens || !out) return PKV_EINVAL;
  if ((phases & kPartitions) && (!q || !k_cache || !v_cache || !block_tables)) return PKV_EINVAL;
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
  a.pb_per_part = partition_blocks > 0
                      ? partition_blocks
                      : auto_partition_blocks(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq);
  a.num_parts = static_cast<int32_t>(ceil_div64(max_blocks_per_seq, a.pb_per_part));
  a.qk_scale = scale * kLog2e;
  if (static_cast<int64_t>(num_kv_heads) * a.head_groups > 65535 || num_seqs > 65535) return PKV_EINVAL;
  if (a.num_parts > 1) {
    const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, a.num_parts);
    if (!workspace || workspace_bytes < need) return PKV_ESMALL;
    const int64_t rows = static_cast<int64_t>(num_seqs) * num_heads * a.num_parts;
    char* ws = const_cast<char*>(static_cast<const char*>(workspace));
    a.ws_o = reinterpret_cast<float*>(ws);
    a.ws_lse = reinterpret_cast<float*>(ws + ceil_div64(rows * head_dim * 4, 256) * 256);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case PKV_BF16:
      return head_dim == 128 ? launch_decode<__bf16, 128>(a, num_seqs, phases, s)
                             : launch_decode<__bf16, 64>(a, num_seqs, phases, s);
    case PKV_F16:
      return head_dim == 128 ? launch_decode<_Float16, 128>(a, num_seqs, phases, s)
                             : launch_decode<_Float16, 64>(a, num_seqs, phases, s);
    case PKV_F32:
      return head_dim == 128 ? launch_decode<float, 128>(a, num_seqs, phases, s)
                             : launch_decode<float, 64>(a, num_seqs, phases, s);
  }
  return PKV_EINVAL;
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

int32_t pkv_version(void) { return 100; }

pkv_status pkv_kv_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                         void* k_cache, void* v_cache, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, pkv_dtype dtype, void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return PKV_EINVAL;
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
                     num_kv_heads, row_bytes, block_size, static_cast<int64_t>(num_blocks) * block_size);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

int32_t pkv_decode_partition_blocks(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t max_blocks_per_seq) {
  return auto_partition_blocks(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq);
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t partition_blocks) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0) return 0;
  const int32_t pb = partition_blocks > 0 ? partition_blocks
                                          : auto_partition_blocks(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq);
  return workspace_bytes_for(num_seqs, num_heads, head_dim, ceil_div64(max_blocks_per_seq, pb));
}

pkv_status pkv_paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      float scale, void* out, pkv_dtype dtype, void* workspace,
                                      size_t workspace_bytes, int32_t partition_blocks, void* stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, out, dtype, workspace, workspace_bytes,
                      partition_blocks, kPartitions | kMerge, stream);
}

pkv_status pkv_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, float scale, void* out, pkv_dtype dtype,
                                 void* workspace, size_t workspace_bytes, int32_t partition_blocks, void* stream) {
  return decode_entry(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, num_blocks, scale, out, dtype, workspace, workspace_bytes,
                      partition_blocks, kPartitions, stream);
}

pkv_status pkv_decode_merge(const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_blocks, void* out,
                            pkv_dtype dtype, void* stream) {
  return decode_entry(nullptr, nullptr, nullptr, nullptr, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                      num_kv_heads, head_dim, block_size, 1, 0.f, out, dtype, workspace, workspace_bytes,
                      partition_blocks, kMerge, stream);
}

}  // extern "C"
