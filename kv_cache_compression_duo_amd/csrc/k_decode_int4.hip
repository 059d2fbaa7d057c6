// Decode step over a 4-bit retrieval cache: split-K attention of retrieval
// heads with the dequantisation folded into MFMA contractions, attention of
// streaming heads over their fp16/bf16 ring, and the log-sum-exp merge.
//
// The pages combine the method with a 4-bit KV cache to reach 3.3M tokens of
// context on one GPU (xllm-io review "DuoAttention: Efficient Long-Context LLM
// Inference with Retrieval and Streaming Heads", section 五 量化组合;
// paperlayer summary of arXiv 2410.10819v1, section 1). The encoding is this
// library's reading: per token, head and 32-channel group g an fp16 scale s
// and zero-point z, x^ = c * s + z with 4-bit codes c.
//
// Exact refactoring used here (no dequantised tensor is formed):
//   q . k^_t = sum_g [ s_tg * sum_{d in g} q_d c_td  +  z_tg * sum_{d in g} q_d ]
//   sum_t p_t v^_td = sum_t (p_t s_tg) c_td + sum_t p_t z_tg        (g = g(d))
// Key codes enter the QK MFMA as bf16 128 + c (exact, one v_perm per pair);
// the accumulator starts at -128 * sum_{d in g} q_d, which removes the offset.
// Value codes enter the PV MFMA as fp16 128 + c (exact: the code shifted into
// the mantissa under a fixed high byte, no fp16 subtraction), against the A
// operand a_t = fp16(p_t s_tg) (11-bit significand: the value and zero-point
// terms of a short row cancel, so bf16 weights would be too coarse). One more
// product of the same A operand against ones gives sum_t a_t per row, and 128
// times it is subtracted at the end: the correction uses the very rounded a_t
// the codes were multiplied by, so the offset cancels in fp32 (fp16 products
// are exact there), at 128 / 7.5 times the accumulator's rounding of the bare
// codes. Q stays bf16 as given.
//
// gfx950 design (v_mfma_f32_16x16x32_bf16 / _f16, one wave = 32 tokens per
// tile, the next tile's loads in flight while the current one is computed):
//   * QK: A = key codes, rows = 16 tokens, k = the 8 channels a lane unpacks
//     from one code word. A lane loads D/8 contiguous bytes of a token row
//     (one 16-byte load for D = 128), i.e. all its channels lie in one
//     32-channel group. B = a block-diagonal Q^T whose 16 columns are
//     (query head h, group g) pairs, zero where the lane's channels are not in
//     group g, so the accumulator column (h, g) collects the group-g partial
//     dot; the groups are then summed with DPP and the scale/zero epilogue
//     runs on every lane without padding waste;
//   * PV: A = p * s_V for the lane's (head, group) row and its 8
//     tokens -- the very tokens and row the QK accumulator left in that lane,
//     so no shuffle is needed -- and B = value codes, whose block layout makes
//     a lane's operands for 4 consecutive 16-channel n-blocks one 16-byte load;
//   * the scale/zero words of the lane's group and tokens are contiguous in
//     the blocked [block][group][32] layout: two 16-byte loads per tile each
//     for K and V;
//   * the running maximum is rescaled only when some lane's maximum grows.
#include "decode_common.hpp"
#include "duo_internal.hpp"
#include "int4_codec.hpp"
#include "split_merge.hpp"

namespace duo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Int4DecodeArgs {
  const uint16_t* q;       // [B][Hq][D] bf16
  const uint16_t* k_new;   // [B][Hkv][D] ring dtype
  const uint16_t* v_new;
  uint16_t* out;           // [B][Hq][D] bf16
  uint8_t* kcodes;         // [B][Hr][cap32][D/2] bytes
  uint8_t* vcodes;         // [B][Hr][cap32/32][16 D] bytes
  uint32_t* ksz;           // [B][Hr][cap32/32][D/32][32] (fp16 s | fp16 z << 16)
  uint32_t* vsz;
  uint16_t* kr;            // ring [B][Hs][S+R][D]
  uint16_t* vr;
  uint32_t* counters;
  float* ml;
  float* acc;
  int Hq, Hkv, Hr, Hs, S, R, max_split;
  int64_t cap32;
  int n;                   // position of the new token (quantised into the cache here),
                           // every sequence unless ragged
  int n_split, split_tokens;
  int ragged;             // sequences hold different counts (use nseq)
  float qscale;            // softmax scale * log2(e)
  // per-sequence positions last: the fields every block reads stay on
  // the first lines of the argument block
  int nseq[kMaxRaggedBatch];  // position of the new token per sequence
};

// 8 nibbles of a word -> 8 16-bit lanes whose low byte is the code and high
// byte is HB (bf16 0x43.. = 128 + c, exact), in the order low nibbles of
// bytes 0..3, then high nibbles.
template <uint32_t HB>
__device__ __forceinline__ u32x4 nib8_to_16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t cb = HB * 0x01010101u;  // selector bytes 4..7 pick from cb
  u32x4 r;
  r.x = __builtin_amdgcn_perm(cb, lo, 0x04010400u);
  r.y = __builtin_amdgcn_perm(cb, lo, 0x04030402u);
  r.z = __builtin_amdgcn_perm(cb, hi, 0x04010400u);
  r.w = __builtin_amdgcn_perm(cb, hi, 0x04030402u);
  return r;
}
__device__ __forceinline__ bf16x8 nib8_to_bf16(uint32_t w) {
  return __builtin_bit_cast(bf16x8, nib8_to_16<0x43u>(w));
}
// 8 nibbles -> 8 fp16 values 128 + c (bits 0x5800 | c << 3, exact), same lane
// order as nib8_to_16: the codes are moved to bits 3..6 of their bytes before
// the high byte 0x58 is inserted.
__device__ __forceinline__ f16x8 nib8_to_f16_128(uint32_t w) {
  const uint32_t lo = (w << 3) & 0x78787878u;
  const uint32_t hi = (w >> 1) & 0x78787878u;
  const uint32_t cb = 0x58585858u;
  u32x4 r;
  r.x = __builtin_amdgcn_perm(cb, lo, 0x04010400u);
  r.y = __builtin_amdgcn_perm(cb, lo, 0x04030402u);
  r.z = __builtin_amdgcn_perm(cb, hi, 0x04010400u);
  r.w = __builtin_amdgcn_perm(cb, hi, 0x04030402u);
  return __builtin_bit_cast(f16x8, r);
}
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// (scale, zero) of a packed word as floats
__device__ __forceinline__ float sz_scale(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w).x;
}
__device__ __forceinline__ float sz_zero(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w).y;
}

// x *= c in the register that holds x. Written as one tied-operand
// instruction so that the rarely taken rescale branch updates the
// accumulators where they are, instead of the compiler copying all of them
// on the path that skips it.
__device__ __forceinline__ float scale_in_place(float x, float c) {
  asm volatile("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(c));
  return x;
}

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// One wave-tile of 32 tokens as a lane holds it.
template <int D>
struct I4Tile {
  static constexpr int KW = D / 32;  // key code words per lane per 16 tokens
  static constexpr int NC = D / 64;  // 16-byte value code loads per lane
  uint32_t k[2][KW];
  u32x4 v[NC];
  u32x4 ks[2], vs[2];
};

// Where one head's arrays are read from: one buffer resource per array (the
// layout check bounds a head's code and scale arrays below 2^31 bytes, so
// 32-bit offsets reach all of them) and this lane's constant byte offsets.
// A tile's own offset is a scalar, so no per-tile vector address is built.
struct I4Src {
  __amdgpu_buffer_rsrc_t k, v, ks, vs;
  uint32_t klane, vlane, slane;
};

template <int D>
__device__ __forceinline__ void load_tile(I4Tile<D>& T, const I4Src& S, int t0) {
  constexpr int NG = D / 32;
  const uint32_t t = (uint32_t)t0;
  // key rows t + 16 hf + n16, bytes q4 * D/8 .. + D/8 of the row
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const uint32_t so = (t + 16 * hf) * (D / 2);
    if constexpr (D == 128) {
      const u32x4 w = buf_ld16_nt(S.k, S.klane, so);
      T.k[hf][0] = w.x; T.k[hf][1] = w.y; T.k[hf][2] = w.z; T.k[hf][3] = w.w;
    } else {
      buf_ld8_nt(S.k, S.klane, so, T.k[hf][0], T.k[hf][1]);
    }
  }
  // value block t/32: 16-byte piece (c4 * 16 + n16) * 4 + q4
  const uint32_t blk = t >> 5;
#pragma unroll
  for (int c4 = 0; c4 < I4Tile<D>::NC; ++c4)
    T.v[c4] = buf_ld16_nt(S.v, S.vlane, blk * 16 * D + c4 * 1024);
  // scale/zero words (blk * NG + gc) * 32 + 4 q4 + 16 hf .. + 3
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    T.ks[hf] = buf_ld16_nt(S.ks, S.slane, blk * NG * 128 + 64 * hf);
    T.vs[hf] = buf_ld16_nt(S.vs, S.slane, blk * NG * 128 + 64 * hf);
  }
}

// Waves per block: two waves per SIMD let one wave's dequantisation overlap
// another's loads (the tile loop is VALU-heavy).
constexpr int kI4Waves = 8;

template <int D, int G, typename RingTag>
__global__ __launch_bounds__(64 * kI4Waves) void decode_int4_kernel(Int4DecodeArgs a) {
  constexpr int NW = kI4Waves;
  constexpr int NG = D / 32;     // channel groups
  constexpr int NCOL = G * NG;   // used MFMA columns (head, group)
  constexpr int NB = D / 16;     // 16-channel n-blocks of the PV product
  static_assert(NCOL <= 16, "G * D / 32 must fit 16 MFMA columns");
  __shared__ BlockRed<D, G, NW> red;
  __shared__ MergeLds<64 * NW> mlds;
  __shared__ int is_last;

  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const bool retrieval = (int)blockIdx.x >= a.Hs;
  const int rb = (int)blockIdx.x - a.Hs;
  const int kvh = retrieval ? rb / a.n_split : a.Hr + (int)blockIdx.x;
  // this sequence's new-token position (sequences may hold different counts;
  // the splits cover the longest, so a shorter one's last splits are empty)
  int n = a.n;
  if (a.ragged) n = a.nseq[b];  // only layers of at most kMaxRaggedBatch sequences

  if (!retrieval) {
    // streaming head: identical to the bf16/fp16 decode path
    constexpr int LPR = D / 8;
    const int lc = lane % LPR;
    float qf[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float t[8];
      unpack8<Bf16Tag>(ld16(a.q + ((int64_t)b * a.Hq + kvh * G + g) * D + lc * 8), t);
#pragma unroll
      for (int c = 0; c < 8; ++c) qf[g][c] = t[c] * a.qscale;
    }
    const uint16_t* knew = a.k_new + ((int64_t)b * a.Hkv + kvh) * D;
    const uint16_t* vnew = a.v_new + ((int64_t)b * a.Hkv + kvh) * D;
    const int hs = kvh - a.Hr;
    const int Wr = a.S + a.R;
    const int nslots = n + 1 < Wr ? n + 1 : Wr;
    const int slot_new = n < a.S ? n : a.S + (n - a.S) % a.R;
    const int64_t hb = (int64_t)b * a.Hs + hs;
    const uint16_t* kr = a.kr + hb * Wr * D;
    const uint16_t* vr = a.vr + hb * Wr * D;
    auto kp = [=](int row) { return row == slot_new ? knew : kr + (int64_t)row * D; };
    auto vp = [=](int row) { return row == slot_new ? vnew : vr + (int64_t)row * D; };
    WaveState<G> st;
    attend_rows<D, G, RingTag, NW>(st, qf, 0, nslots, kp, vp);
    if (threadIdx.x < LPR) {
      st16(a.kr + (hb * Wr + slot_new) * D + threadIdx.x * 8, ld16(knew + threadIdx.x * 8));
      st16(a.vr + (hb * Wr + slot_new) * D + threadIdx.x * 8, ld16(vnew + threadIdx.x * 8));
    }
    block_merge<D, G, NW>(red, st);
    for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
      int g = i / D, dd = i % D;
      a.out[((int64_t)b * a.Hq + kvh * G + g) * D + dd] =
          (uint16_t)f2bf(red.acc[0][g][dd] / red.L[g]);
    }
    return;
  }

  // ---------------------------------------------------------------- retrieval
  const int split = rb % a.n_split;
  const int r0 = split * a.split_tokens;
  const int r_end = r0 + a.split_tokens < n + 1 ? r0 + a.split_tokens : n + 1;
  // the split holding position n also takes the new token, which it quantises
  // itself (below); its cache rows end at n
  const bool has_new = r0 <= n && r_end == n + 1;  // splits past n are empty
  const int r1 = has_new ? n : r_end;
  const int64_t hb = (int64_t)b * a.Hr + kvh;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int hc = n16 / NG, gc = n16 % NG;  // this lane's (head, group) column
  const bool col_ok = n16 < NCOL;
  constexpr int KW = I4Tile<D>::KW;
  // group of the channels this lane unpacks from a key row (D/4 per lane)
  const int lane_group = q4 * D / 128;

  // block-diagonal Q^T operands (one per code word) and per-column q sums
  bf16x8 qop[KW];
  float qsum;
  {
    const uint16_t* qh = a.q + ((int64_t)b * a.Hq + kvh * G + (col_ok ? hc : 0)) * D;
    // sum of the column's group of Q (32 channels: 4 lanes x 8)
    const u32x4 graw = ld16(qh + 32 * gc + 8 * q4);
    float s8 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s8 += __uint_as_float((uint32_t)half_of(graw, i) << 16);
    s8 += __shfl_xor(s8, 16, 64);
    s8 += __shfl_xor(s8, 32, 64);
    qsum = col_ok ? s8 : 0.0f;
    // B operand of code word j: channels q4*D/4 + 8j + {0,2,4,6,1,3,5,7}
    constexpr int perm8[8] = {0, 2, 4, 6, 1, 3, 5, 7};
    const bool diag = col_ok && lane_group == gc;
#pragma unroll
    for (int j = 0; j < KW; ++j) {
      const u32x4 raw = ld16(qh + q4 * (D / 4) + 8 * j);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t bits = diag ? half_of(raw, perm8[i]) : (uint16_t)0;
        qop[j][i] = __builtin_bit_cast(__bf16, bits);
      }
    }
  }
  const float qoff = -128.0f * qsum;
  const float qscale = a.qscale;

  I4Src src;
  {
    const uint32_t code_bytes = (uint32_t)(a.cap32 * (D / 2));
    const uint32_t sz_bytes = (uint32_t)(a.cap32 * NG * 4);
    src.k = wave_rsrc(a.kcodes + hb * a.cap32 * (D / 2), code_bytes);
    src.v = wave_rsrc(a.vcodes + hb * a.cap32 * (D / 2), code_bytes);
    src.ks = wave_rsrc(a.ksz + hb * a.cap32 * NG, sz_bytes);
    src.vs = wave_rsrc(a.vsz + hb * a.cap32 * NG, sz_bytes);
    src.klane = (uint32_t)(n16 * (D / 2) + q4 * (D / 8));
    src.vlane = (uint32_t)((n16 * 4 + q4) * 16);
    src.slane = (uint32_t)((gc * 32 + 4 * q4) * 4);
  }

  float m_run = -INFINITY, l_run = 0.0f, zacc = 0.0f;
  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // row sums of the PV A operand (p * s_V rounded to fp16), taken by one more
  // product against ones: the value codes enter as 128 + c, so 128 times
  // this sum is subtracted from every channel of the row at the end
  f32x4 asum = f32x4{0.f, 0.f, 0.f, 0.f};
  const f16x8 ones8 = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                       (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};

  // FULL: all 32 tokens of the tile are below r1 (no masking, no stale
  // scale words); only the last tile of a split can be partial.
  auto compute = [&](const I4Tile<D>& T, int t0, auto full_c) {
    constexpr bool full = decltype(full_c)::value;
    // ---- scores: per-group dots on MFMA, scale/zero epilogue, group sum ----
    float sc[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 pk = f32x4{qoff, qoff, qoff, qoff};
#pragma unroll
      for (int j = 0; j < KW; ++j)
        pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nib8_to_bf16(T.k[hf][j]), qop[j], pk, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t w = word_of(T.ks[hf], r);
        float v = fmaf(sz_scale(w), pk[r], sz_zero(w) * qsum);
        if constexpr (NG >= 2) v += dpp<0xB1>(v);  // sum over the NG group lanes
        if constexpr (NG >= 4) v += dpp<0x4E>(v);
        sc[hf][r] = v;
      }
    }
    if constexpr (!full) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + 16 * hf + 4 * q4 + r >= r1) sc[hf][r] = -INFINITY;
    }
    // ---- online softmax for this lane's head (scores in units of qscale) ----
    float tm = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
    tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
    if (__builtin_amdgcn_ballot_w64(tm > m_run)) {
      // some head's maximum grew (every tile holds a valid token, so tm is
      // finite and the first tile always lands here)
      const float mn = fmaxf(m_run, tm);
      const float corr = fast_exp2((m_run - mn) * qscale);
      m_run = mn;
      l_run *= corr;
      zacc *= corr;
      // output row 4*q4 + r of the PV product is column (head, group)
      // ((4q4 + r) / NG, (4q4 + r) % NG)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float cr = __shfl(corr, ((4 * q4 + r) / NG) * NG, 64);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[nb][r] = scale_in_place(o[nb][r], cr);
        asum[r] = scale_in_place(asum[r], cr);
      }
    }
    const float mq = m_run * qscale;
    float p[2][4], ls = 0.0f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[hf][r] = fast_exp2(fmaf(sc[hf][r], qscale, -mq));
        ls += p[hf][r];
      }
    l_run += ls;
    // ---- PV: A = p * s_V (fp16) for this lane's (head, group) row ----
    f16x8 pa;
    float zt = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int hf = i >> 2, r = i & 3;
      const uint32_t w = word_of(T.vs[hf], r);
      float s = sz_scale(w), z = sz_zero(w);
      if constexpr (!full) {
        // tokens past the end carry stale scale words; p is 0 there
        const bool ok = p[hf][r] > 0.0f;
        s = ok ? s : 0.0f;
        z = ok ? z : 0.0f;
      }
      pa[i] = (_Float16)(p[hf][r] * s);
      zt = fmaf(p[hf][r], z, zt);
    }
    zacc += zt;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          pa, nib8_to_f16_128(word_of(T.v[nb / 4], nb % 4)), o[nb], 0, 0, 0);
    asum = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, ones8, asum, 0, 0, 0);
  };
  // Ping-pong tiles: the next tile's loads are issued before the current tile
  // is computed. Tiles past the range are clamped to the last tile (a cached
  // re-read, never computed), so every load stays inside the allocation.
  const int last_tile = ((r1 - 1) >> 5) << 5;
  auto clamp = [&](int t) { return t < last_tile ? t : last_tile; };
  constexpr int stride = NW * 32;
  int t0 = r0 + wave * 32;
  if (t0 < r1) {
    I4Tile<D> ta, tb;
    load_tile<D>(ta, src, t0);
    auto step = [&](const I4Tile<D>& T, int t) {
      if (t + 32 <= r1) compute(T, t, BoolC<true>{});
      else compute(T, t, BoolC<false>{});
    };
    for (;;) {
      const int t1 = t0 + stride;
      load_tile<D>(tb, src, clamp(t1));
      step(ta, t0);
      if (t1 >= r1) break;
      t0 = t1 + stride;
      load_tile<D>(ta, src, clamp(t0));
      step(tb, t1);
      if (t0 >= r1) break;
    }
  }

  // ---- the new token ---------------------------------------------------------
  // Quantised here exactly as the append kernel does (lanes 0..D/8-1 of wave 0
  // encode K, lanes 32.. encode V, 8 channels each, quads = 32-channel
  // groups); its codes and scale/zero words are written for later steps. No
  // block of this launch reads row n as data: the 32-token tile holding it
  // belongs to this split only and is masked past the cache rows, and the one
  // value-code byte it shares with token n - 16 keeps that token's nibble.
  // It enters the block merge from its dequantised values fma(c, s, z) as one
  // more entry: score q . k^ per head, weight 1, values v^.
  __shared__ float new_m[G];
  __shared__ float new_acc[G][D];
  if (has_new && wave == 0) {
    constexpr int CH = D / 8;  // 8-channel chunks of a row
    const bool vside = lane >= 32;
    const bool act = (lane & 31) < CH;
    const int c = act ? (lane & 31) : 0;  // idle quads duplicate chunks 0..3
    const uint16_t* src = (vside ? a.v_new : a.k_new) + ((int64_t)b * a.Hkv + kvh) * D + 8 * c;
    uint32_t codes, sz;
    encode_group_part<RingTag>(ld16(src), &codes, &sz);
    if (act) {
      const int64_t w = ((hb * (a.cap32 / 32) + n / 32) * NG + c / 4) * 32 + n % 32;
      if (!vside) {
        reinterpret_cast<uint32_t*>(a.kcodes)[(hb * a.cap32 + n) * CH + c] = codes;
        if ((c & 3) == 0) a.ksz[w] = sz;
      } else {
        if ((c & 3) == 0) a.vsz[w] = sz;
        // token n is nibble n / 16 % 2 of byte position n % 16 of its block
        const int m16 = n % 16;
        const bool hi = (n % 32) >= 16;
        uint8_t* vb = a.vcodes + (hb * (a.cap32 / 32) + n / 32) * 16 * D +
                      16 * (4 * (16 * (c / 8) + 8 * (c % 2)) + m16 / 4) + 4 * ((c % 8) / 2) +
                      m16 % 4;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint8_t* dst = vb + 64 * j;
          const uint32_t nib = (codes >> (4 * j)) & 0xFu;
          const uint32_t old = *dst;
          *dst = (uint8_t)(hi ? (old & 0x0Fu) | (nib << 4) : (old & 0xF0u) | nib);
        }
      }
    }
    float xh[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xh[j] = decode_code(codes, sz, j);
    // per-head dot q . k^ over the K lanes (lanes 0..31; others add 0)
    float dots[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float qv[8];
      unpack8<Bf16Tag>(ld16(a.q + ((int64_t)b * a.Hq + kvh * G + g) * D + 8 * c), qv);
      float d = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) d = fmaf(qv[j], xh[j], d);
      dots[g] = (!vside && act) ? d : 0.0f;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) dots[g] += __shfl_xor(dots[g], off, 64);
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) new_m[g] = dots[g] * a.qscale;  // log2 units
    }
    if (vside && act) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) new_acc[g][8 * c + j] = xh[j];
    }
  }

  // ---- wave totals -> LDS --------------------------------------------------
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  zacc += __shfl_xor(zacc, 16, 64);
  zacc += __shfl_xor(zacc, 32, 64);
  const bool wave_live = r0 + wave * 32 < r1;
  if (lane < NCOL && gc == 0 && lane / NG < G) {
    red.m[wave][hc] = wave_live ? m_run * qscale : -INFINITY;
    red.l[wave][hc] = wave_live ? l_run : 0.0f;
  }
  // zero-point term of output row 4*q4 + r, held by lane (row) --
  // fetched with every lane active
  float zrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) zrow[r] = __shfl(zacc, 4 * q4 + r, 64);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * q4 + r;
      const int h = row / NG, g = row % NG;
      if (row < NCOL && g == nb / 2)
        red.acc[wave][h][16 * nb + n16] =
            wave_live ? fmaf(-128.0f, asum[r], o[nb][r] + zrow[r]) : 0.0f;
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = red.m[0][g];
    for (int w = 1; w < NW; ++w) M = fmaxf(M, red.m[w][g]);
    if (has_new) M = fmaxf(M, new_m[g]);
    float Lsum = 0.0f;
    for (int w = 0; w < NW; ++w)
      Lsum += red.m[w][g] == -INFINITY ? 0.0f : red.l[w][g] * fast_exp2(red.m[w][g] - M);
    if (has_new) Lsum += fast_exp2(new_m[g] - M);
    red.M[g] = M;
    red.L[g] = Lsum;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int g = i / D, dd = i % D;
    float s = 0.0f;
    for (int w = 0; w < NW; ++w)
      if (red.m[w][g] != -INFINITY) s += red.acc[w][g][dd] * fast_exp2(red.m[w][g] - red.M[g]);
    if (has_new) s += new_acc[g][dd] * fast_exp2(new_m[g] - red.M[g]);
    red.acc[0][g][dd] = s;  // each (g, dd) is read and written by one thread only
  }
  __syncthreads();

  // ---- publish the split's partial, last block merges ------------------------
  const int64_t pbase = (hb * G) * a.max_split;
  const PartialView pv = partial_view<D, G>(a.ml + pbase * 2, a.acc + pbase * D, a.max_split);
  publish_partial<D, G>(pv, a.max_split, split, &red.acc[0][0][0], red.M, red.L);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t prev = __hip_atomic_fetch_add(a.counters + hb, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == (uint32_t)(a.n_split - 1));
  }
  __syncthreads();
  if (!is_last) return;
  merge_splits<D, G, 64 * NW>(mlds, pv, a.max_split, a.n_split,
                     a.out + ((int64_t)b * a.Hq + kvh * G) * D);
  if (threadIdx.x == 0)
    __hip_atomic_store(a.counters + hb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int G, typename RingTag>
static hipError_t launch_i4(Int4DecodeArgs a, int B, int64_t rows, int st, int max_split,
                            hipStream_t s) {
  a.split_tokens = st;
  a.n_split = a.Hr > 0 ? (int)((rows + st - 1) / st) : 0;
  if (a.n_split > max_split) return hipErrorInvalidValue;
  dim3 grid((unsigned)(a.Hr * a.n_split + a.Hs), (unsigned)B);
  decode_int4_kernel<D, G, RingTag><<<grid, 64 * kI4Waves, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, typename RingTag>
static hipError_t launch_i4_g(int G, const Int4DecodeArgs& a, int B, int64_t rows, int st,
                              int max_split, hipStream_t s) {
  switch (G) {
    case 1: return launch_i4<D, 1, RingTag>(a, B, rows, st, max_split, s);
    case 2: return launch_i4<D, 2, RingTag>(a, B, rows, st, max_split, s);
    case 4: return launch_i4<D, 4, RingTag>(a, B, rows, st, max_split, s);
    default:
      if constexpr (D == 64) return launch_i4<D, 8, RingTag>(a, B, rows, st, max_split, s);
      return hipErrorInvalidValue;  // G = 8 with D = 128 exceeds 16 columns
  }
}

hipError_t launch_decode_int4(const duo_layer* L, const void* q, const void* k_new,
                              const void* v_new, void* out, hipStream_t s) {
  const duo_layer_desc& d = L->d;
  // one launch: the block whose split holds position n quantises the new
  // token into the 4-bit cache and attends to it
  Int4DecodeArgs a;
  WsView ws = ws_view(L);
  a.q = static_cast<const uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.out = static_cast<uint16_t*>(out);
  a.kcodes = reinterpret_cast<uint8_t*>(L->rbuf + L->lay.k_offset);
  a.vcodes = reinterpret_cast<uint8_t*>(L->rbuf + L->lay.v_offset);
  a.ksz = reinterpret_cast<uint32_t*>(L->rbuf + L->lay.k_sz_offset);
  a.vsz = reinterpret_cast<uint32_t*>(L->rbuf + L->lay.v_sz_offset);
  a.kr = reinterpret_cast<uint16_t*>(L->sbuf + L->lay.ring_k_offset);
  a.vr = reinterpret_cast<uint16_t*>(L->sbuf + L->lay.ring_v_offset);
  a.counters = ws.counters;
  a.ml = ws.ml;
  a.acc = ws.acc;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.Hr = L->Hr;
  a.Hs = L->Hs;
  a.S = d.sink;
  a.R = d.recent;
  a.max_split = L->max_split;
  a.cap32 = cap32_of(d.retrieval_capacity);
  a.n = (int)L->n;
  a.ragged = L->ragged ? 1 : 0;
  // ragged positions travel in the arguments: larger batches come in slices
  if (L->ragged && d.batch > kMaxRaggedBatch) return hipErrorInvalidValue;
  for (int b = 0; b < d.batch && b < kMaxRaggedBatch; ++b) a.nseq[b] = (int)L->nseq[b];
  a.qscale = d.softmax_scale * kLog2e;
  const int64_t rows = L->n + 1;  // the longest sequence
  const int B = d.batch;
  const int st = decode_split_tokens(L, rows, 32, L->cus);
  const int ms = L->max_split;
  if (d.head_dim == 128) {
    if (d.kv_dtype == DUO_FP16) return launch_i4_g<128, Fp16Tag>(L->G, a, B, rows, st, ms, s);
    return launch_i4_g<128, Bf16Tag>(L->G, a, B, rows, st, ms, s);
  }
  if (d.kv_dtype == DUO_FP16) return launch_i4_g<64, Fp16Tag>(L->G, a, B, rows, st, ms, s);
  return launch_i4_g<64, Bf16Tag>(L->G, a, B, rows, st, ms, s);
}

}  // namespace duo
