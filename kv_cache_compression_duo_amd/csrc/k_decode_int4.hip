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
// Key codes enter the QK MFMA as bf16 128 + c (exact, one v_perm per pair)
// and the offset is removed from the per-group dot afterwards. Value codes
// enter the PV MFMA as exact fp16 c ((1024 + c) - 1024 with packed fp16 adds),
// so the rounded p * s_V operand (fp16, 11-bit significand) appears in no
// other term and needs no matching correction. Q stays bf16 as given.
//
// gfx950 design (v_mfma_f32_16x16x32_bf16, one wave = 32 tokens per tile):
//   * QK: A = key codes (16 tokens x 32 channels of group g), B = a
//     block-diagonal Q^T whose 16 columns are (query head h, group g') pairs,
//     zero unless g' = g. Four MFMAs (one per group) fill all 16 columns with
//     the per-group partial dots, so the scale/zero epilogue runs on every
//     lane without padding waste; the groups are then summed with DPP;
//   * PV (fp16 MFMA): A = p * s_V for the lane's (head, group) row and its 8
//     tokens -- the
//     very tokens and row the QK accumulator left in that lane, so no shuffle
//     is needed -- and B = value codes. Value codes are stored transposed in
//     32-token blocks, [channel][16 bytes], byte m holding tokens m (low
//     nibble) and m + 16 (high nibble), which is exactly the B operand order;
//   * key codes keep the token-major layout (byte b of a row: channel 2b low
//     nibble, 2b + 1 high); the v_perm unpacking yields channels in the order
//     0,2,4,6,1,3,5,7 of each 8-channel word and Q is loaded in that order.
#include <stdlib.h>

#include "decode_common.hpp"
#include "duo_internal.hpp"
#include "split_merge.hpp"

namespace duo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Int4DecodeArgs {
  const uint16_t* q;       // [B][Hq][D] bf16
  const uint16_t* k_new;   // [B][Hkv][D] ring dtype
  const uint16_t* v_new;
  uint16_t* out;           // [B][Hq][D] bf16
  const uint32_t* kcodes;  // [B][Hr][cap32][D/8] words
  const uint32_t* vcodes;  // [B][Hr][cap32/32][D][4] words
  const uint32_t* ksz;     // [B][Hr][cap32][D/32] (fp16 s | fp16 z << 16)
  const uint32_t* vsz;
  uint16_t* kr;            // ring [B][Hs][S+R][D]
  uint16_t* vr;
  uint32_t* counters;
  float* ml;
  float* acc;
  int Hq, Hkv, Hr, Hs, S, R, max_split;
  int64_t cap32;
  int n;                   // position of the new token (already in the 4-bit cache)
  int n_split, split_tokens;
  float qscale;            // softmax scale * log2(e)
};

// 8 nibbles -> 16-bit floats (OFF + c) with high byte HB (bf16 0x43.. = 128 + c,
// fp16 0x64.. = 1024 + c, both exact), in the order low nibbles of bytes
// 0..3, then high nibbles.
template <uint32_t HB>
__device__ __forceinline__ u32x4 nib8_to_16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t cb = HB * 0x01010101u;
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
// 8 nibbles -> exact fp16 codes c: (1024 + c) - 1024 with packed fp16 adds.
__device__ __forceinline__ f16x8 nib8_to_f16(uint32_t w) {
  const f16x8 biased = __builtin_bit_cast(f16x8, nib8_to_16<0x64u>(w));
  const f16x8 off = {(_Float16)1024.0f, (_Float16)1024.0f, (_Float16)1024.0f, (_Float16)1024.0f,
                     (_Float16)1024.0f, (_Float16)1024.0f, (_Float16)1024.0f, (_Float16)1024.0f};
  return biased - off;
}

__device__ __forceinline__ float h2f_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float h2f_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

template <int D, int G, typename RingTag>
__global__ __launch_bounds__(256) void decode_int4_kernel(Int4DecodeArgs a) {
  constexpr int NG = D / 32;     // channel groups
  constexpr int NCOL = G * NG;   // used MFMA columns (head, group)
  constexpr int NB = D / 16;     // 16-channel n-blocks of the PV product
  constexpr int W = D / 8;       // code words per token row
  static_assert(NCOL <= 16, "G * D / 32 must fit 16 MFMA columns");
  __shared__ BlockRed<D, G> red;
  __shared__ MergeLds mlds;
  __shared__ int is_last;

  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool retrieval = (int)blockIdx.x >= a.Hs;
  const int rb = (int)blockIdx.x - a.Hs;
  const int kvh = retrieval ? rb / a.n_split : a.Hr + (int)blockIdx.x;

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
    const int nslots = a.n + 1 < Wr ? a.n + 1 : Wr;
    const int slot_new = a.n < a.S ? a.n : a.S + (a.n - a.S) % a.R;
    const int64_t hb = (int64_t)b * a.Hs + hs;
    const uint16_t* kr = a.kr + hb * Wr * D;
    const uint16_t* vr = a.vr + hb * Wr * D;
    auto kp = [=](int row) { return row == slot_new ? knew : kr + (int64_t)row * D; };
    auto vp = [=](int row) { return row == slot_new ? vnew : vr + (int64_t)row * D; };
    WaveState<G> st;
    attend_rows<D, G, RingTag>(st, qf, 0, nslots, kp, vp);
    if (threadIdx.x < LPR) {
      st16(a.kr + (hb * Wr + slot_new) * D + threadIdx.x * 8, ld16(knew + threadIdx.x * 8));
      st16(a.vr + (hb * Wr + slot_new) * D + threadIdx.x * 8, ld16(vnew + threadIdx.x * 8));
    }
    block_merge<D, G>(red, st);
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
  const int r1 = r0 + a.split_tokens < a.n + 1 ? r0 + a.split_tokens : a.n + 1;
  const int64_t hb = (int64_t)b * a.Hr + kvh;
  const int n16 = lane & 15, q4 = lane >> 4;
  const int hc = n16 / NG, gc = n16 % NG;  // this lane's (head, group) column
  const bool col_ok = n16 < NCOL;

  // block-diagonal Q^T operands (one per group) and per-column q sums
  bf16x8 qop[NG];
  float qsum;
  {
    const uint16_t* qh = a.q + ((int64_t)b * a.Hq + kvh * G + (col_ok ? hc : 0)) * D;
    const u32x4 raw = ld16(qh + 32 * gc + 8 * q4);  // channels 32gc + 8q4 .. +7
    constexpr int perm8[8] = {0, 2, 4, 6, 1, 3, 5, 7};
    float s8 = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s8 += __uint_as_float((uint32_t)half_of(raw, i) << 16);
    s8 += __shfl_xor(s8, 16, 64);
    s8 += __shfl_xor(s8, 32, 64);
    qsum = col_ok ? s8 : 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t bits = (col_ok && g == gc) ? half_of(raw, perm8[i]) : (uint16_t)0;
        qop[g][i] = __builtin_bit_cast(__bf16, bits);
      }
    }
  }
  const float qs128 = 128.0f * qsum;

  const uint32_t* kc = a.kcodes + hb * a.cap32 * W;
  const uint32_t* vc = a.vcodes + hb * a.cap32 * (D / 2) / 4;
  const uint32_t* ks = a.ksz + hb * a.cap32 * NG;
  const uint32_t* vs = a.vsz + hb * a.cap32 * NG;

  float m_run = -INFINITY, l_run = 0.0f, zacc = 0.0f;
  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t0 = r0 + wave * 32; t0 < r1; t0 += kWaves * 32) {
    // ---- loads (all inside the 32-token-aligned allocation) ----
    uint32_t kw[2][NG], vw[NB], kszw[2][4], vszw[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        kw[hf][g] = __builtin_nontemporal_load(kc + (int64_t)(t0 + 16 * hf + n16) * W + 4 * g + q4);
    const uint32_t* vblk = vc + (int64_t)(t0 >> 5) * D * 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      vw[nb] = __builtin_nontemporal_load(vblk + (16 * nb + n16) * 4 + q4);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * hf + 4 * q4 + r;
        kszw[hf][r] = ks[(int64_t)t * NG + gc];
        vszw[hf][r] = vs[(int64_t)t * NG + gc];
      }
    // ---- scores: per-group dots on MFMA, scale/zero epilogue, group sum ----
    float sc[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4 pk = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < NG; ++g)
        pk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nib8_to_bf16(kw[hf][g]), qop[g], pk, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = h2f_lo(kszw[hf][r]), z = h2f_hi(kszw[hf][r]);
        float v = fmaf(s, pk[r] - qs128, z * qsum);
        if constexpr (NG >= 2) v += dpp<0xB1>(v);  // sum over the NG group lanes
        if constexpr (NG >= 4) v += dpp<0x4E>(v);
        const int t = t0 + 16 * hf + 4 * q4 + r;
        sc[hf][r] = t < r1 ? v * a.qscale : -INFINITY;
      }
    }
    // ---- online softmax for this lane's head ----
    float tm = sc[0][0];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r = 0; r < 4; ++r) tm = fmaxf(tm, sc[hf][r]);
    tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
    tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
    const float mn = fmaxf(m_run, tm);  // finite: every tile has a valid token
    const float corr = fast_exp2(m_run - mn);
    m_run = mn;
    float p[2][4], ls = 0.0f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[hf][r] = fast_exp2(sc[hf][r] - mn);
        ls += p[hf][r];
      }
    l_run = l_run * corr + ls;
    // ---- PV: A = p * s_V (fp16) for this lane's (head, group) row ----
    f16x8 pa;
    float zt = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int hf = i >> 2, r = i & 3;
      const uint32_t w = vszw[hf][r];
      const bool ok = p[hf][r] > 0.0f;  // masked tokens may carry stale scales
      const float s = ok ? h2f_lo(w) : 0.0f, z = ok ? h2f_hi(w) : 0.0f;
      pa[i] = (_Float16)(p[hf][r] * s);
      zt = fmaf(p[hf][r], z, zt);
    }
    zacc = zacc * corr + zt;
    // corr of the head whose rows this lane accumulates in the PV output:
    // output row 4*q4 + r is column (head, group) = ((4q4+r)/NG, (4q4+r)%NG)
    float corr_row[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hrow = (4 * q4 + r) / NG;
      corr_row[r] = __shfl(corr, hrow * NG, 64);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o[nb][r] *= corr_row[r];
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, nib8_to_f16(vw[nb]), o[nb], 0, 0, 0);
    }
  }

  // ---- wave totals -> LDS --------------------------------------------------
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  zacc += __shfl_xor(zacc, 16, 64);
  zacc += __shfl_xor(zacc, 32, 64);
  const bool wave_live = r0 + wave * 32 < r1;
  if (lane < NCOL && gc == 0 && lane / NG < G) {
    red.m[wave][hc] = wave_live ? m_run : -INFINITY;
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
        red.acc[wave][h][16 * nb + n16] = wave_live ? o[nb][r] + zrow[r] : 0.0f;
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = red.m[0][g];
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red.m[w][g]);
    float Lsum = 0.0f;
    for (int w = 0; w < kWaves; ++w)
      Lsum += red.m[w][g] == -INFINITY ? 0.0f : red.l[w][g] * fast_exp2(red.m[w][g] - M);
    red.M[g] = M;
    red.L[g] = Lsum;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int g = i / D, dd = i % D;
    float s = 0.0f;
    for (int w = 0; w < kWaves; ++w)
      if (red.m[w][g] != -INFINITY) s += red.acc[w][g][dd] * fast_exp2(red.m[w][g] - red.M[g]);
    red.acc[0][g][dd] = s;  // each (g, dd) is read and written by one thread only
  }
  __syncthreads();

  // ---- publish the split's partial, last block merges ------------------------
  const int64_t pbase = (hb * G) * a.max_split;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int g = i / D, dd = i % D;
    __hip_atomic_store(a.acc + (pbase + (int64_t)g * a.max_split + split) * D + dd,
                       red.acc[0][g][dd], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float* mlp = a.ml + (pbase + (int64_t)g * a.max_split + split) * 2;
    __hip_atomic_store(mlp, red.M[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(mlp + 1, red.L[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t prev = __hip_atomic_fetch_add(a.counters + hb, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == (uint32_t)(a.n_split - 1));
  }
  __syncthreads();
  if (!is_last) return;
  merge_splits<D, G>(mlds, a.ml + pbase * 2, a.acc + pbase * D, a.max_split, a.n_split,
                     a.out + ((int64_t)b * a.Hq + kvh * G) * D);
  if (threadIdx.x == 0)
    __hip_atomic_store(a.counters + hb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static int env_split_tokens_int4() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("DUO_DECODE_SPLIT_TOKENS");
    v = e ? atoi(e) : 0;
    if (v < 0) v = 0;
  }
  return v;
}

template <typename K>
static int resident_blocks_of(K kernel) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, 256, 0) != hipSuccess ||
      cus <= 0 || per <= 0)
    return 512;
  return cus * per;
}

template <int D, int G, typename RingTag>
static hipError_t launch_i4(Int4DecodeArgs a, int B, int64_t rows, int max_split,
                            hipStream_t s) {
  int st = env_split_tokens_int4();
  if (st <= 0 && a.Hr > 0) {
    static int resident = 0;
    if (!resident) resident = resident_blocks_of(decode_int4_kernel<D, G, RingTag>);
    int slots = resident / B - a.Hs;
    int per_head = slots / a.Hr;
    if (per_head < 1) per_head = 1;
    int64_t t = (rows + per_head - 1) / per_head;
    st = (int)((t + 31) / 32 * 32);
  }
  if (st < kMinSplitTokens) st = kMinSplitTokens;
  st = (st + 31) / 32 * 32;
  a.split_tokens = st;
  a.n_split = (int)((rows + st - 1) / st);
  if (a.n_split > max_split) return hipErrorInvalidValue;
  dim3 grid((unsigned)(a.Hr * a.n_split + a.Hs), (unsigned)B);
  decode_int4_kernel<D, G, RingTag><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int D, typename RingTag>
static hipError_t launch_i4_g(int G, const Int4DecodeArgs& a, int B, int64_t rows,
                              int max_split, hipStream_t s) {
  switch (G) {
    case 1: return launch_i4<D, 1, RingTag>(a, B, rows, max_split, s);
    case 2: return launch_i4<D, 2, RingTag>(a, B, rows, max_split, s);
    case 4: return launch_i4<D, 4, RingTag>(a, B, rows, max_split, s);
    default:
      if constexpr (D == 64) return launch_i4<D, 8, RingTag>(a, B, rows, max_split, s);
      return hipErrorInvalidValue;  // G = 8 with D = 128 exceeds 16 columns
  }
}

hipError_t launch_decode_int4(const duo_layer* L, const void* q, const void* k_new,
                              const void* v_new, void* out, hipStream_t s) {
  const duo_layer_desc& d = L->d;
  // the new token goes into the 4-bit cache first (append, then attend)
  hipError_t e = launch_append_cache(L, k_new, v_new, 1, s);
  if (e != hipSuccess) return e;
  Int4DecodeArgs a;
  WsView ws = ws_view(L);
  a.q = static_cast<const uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.out = static_cast<uint16_t*>(out);
  a.kcodes = reinterpret_cast<const uint32_t*>(L->rbuf + L->lay.k_offset);
  a.vcodes = reinterpret_cast<const uint32_t*>(L->rbuf + L->lay.v_offset);
  a.ksz = reinterpret_cast<const uint32_t*>(L->rbuf + L->lay.k_sz_offset);
  a.vsz = reinterpret_cast<const uint32_t*>(L->rbuf + L->lay.v_sz_offset);
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
  a.qscale = d.softmax_scale * kLog2e;
  const int64_t rows = L->n + 1;
  const int B = d.batch;
  if (d.head_dim == 128) {
    if (d.kv_dtype == DUO_FP16) return launch_i4_g<128, Fp16Tag>(L->G, a, B, rows, L->max_split, s);
    return launch_i4_g<128, Bf16Tag>(L->G, a, B, rows, L->max_split, s);
  }
  if (d.kv_dtype == DUO_FP16) return launch_i4_g<64, Fp16Tag>(L->G, a, B, rows, L->max_split, s);
  return launch_i4_g<64, Bf16Tag>(L->G, a, B, rows, L->max_split, s);
}

}  // namespace duo
