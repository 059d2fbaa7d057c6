// Tiled softmax attention on bf16 MFMA for the prefill paths and the
// gate-blended identification forward.
//
// What is computed (xllm-io review "DuoAttention: Efficient Long-Context LLM
// Inference with Retrieval and Streaming Heads", section 三 核心公式):
//   retrieval heads: softmax over keys j <= i (causal) of scale * q_i . k_j;
//   streaming heads: the same under the Lambda mask, keys j <= i with
//     j < sink or i - j < recent;
//   mixed (identification) forward: alpha * full + (1 - alpha) * streaming
//     with one alpha per KV head (same section, 混合注意力; paperlayer summary
//     of arXiv 2410.10819v1, section 2).
// Prefill is chunked: a chunk's retrieval heads attend over the full cache
// (the chunk already appended), its streaming heads over the ring as it was
// before the chunk plus the chunk itself, so activation memory scales with the
// chunk (xllm-io review, section 三 预填充阶段; paperlayer summary, section 2
// Chunked Pre-filling). The pages run this step with FlashAttention-2 on A100;
// the kernel below is a gfx950 design of the same exact computation.
//
// gfx950 design:
//   * a block is 8 waves; a wave owns 32 query rows (32 tokens of one query
//     head). The HB heads of a block share one KV head (GQA grouping), so one
//     K/V tile in LDS serves 8 waves of query rows; half the waves stage K and
//     half V;
//   * the mixed forward runs in two phases over one tile pipeline and one
//     softmax state: the Lambda tiles (sinks and the window band, a few per
//     query tile) first, folded into (1 - alpha) * O / l kept as bf16 pairs,
//     then all causal tiles as in retrieval mode (the band's QK products are
//     computed twice; two sets of accumulators would halve the occupancy);
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16. In this
//     orientation a lane holds one query's scores, so the softmax needs one
//     cross-lane exchange per tile, and the score accumulator is directly the
//     B operand of the PV product (keys permuted inside each 16-key slice,
//     which a sum over keys does not see);
//   * K tiles are stored row-major in LDS (rows padded by 16 bytes), V tiles
//     transposed (d-major) with 4-key chunks paired and XOR-swizzled by d, so
//     that both MFMA operands are read with one ds_read_b128 each;
//   * the next tile's global loads are in flight while the current tile is
//     computed; query tiles are launched longest-first (causal imbalance).
#include "device_common.hpp"
#include "duo_internal.hpp"

namespace duo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Kernel modes; the _BLOCK variants take the streaming part of the
// two-phase modes under the block-sparse Lambda mask.
enum {
  MODE_RETRIEVAL = 0,
  MODE_STREAMING = 1,
  MODE_MIXED = 2,
  MODE_GRAD = 3,
  MODE_MIXED_BLOCK = 4,
  MODE_GRAD_BLOCK = 5
};

struct AttnArgs {
  const uint16_t* q;     // [B][T][Hq][D]
  uint16_t* out;         // [B][T][Hq][D]
  const uint16_t* k_in;  // chunk / sequence K, V [B][T][Hkv][D]
  const uint16_t* v_in;
  const uint16_t* kc;    // retrieval cache [B][Hr][cap][D]
  const uint16_t* vc;
  const uint16_t* kr;    // ring [B][Hs][S+R][D]
  const uint16_t* vr;
  const float* alpha;    // [Hkv] (mixed)
  const uint16_t* dout;  // [B][T][Hq][D] bf16 (gate gradient)
  float* partial;        // [B][head groups][query tiles] (gate gradient)
  int T, Hq, Hkv, Hr, Hs, G, S, R;
  int64_t cap;
  int n;         // absolute position of token 0 of the chunk (0 for mixed)
  int n_qtiles;  // query token tiles
  int kv_base;   // first KV head handled by the launch
  int tiles_in_y;  // grid (head groups, query tiles) rather than (query tiles, head groups)
  float scale_log2;
};

constexpr int kBN = 64;  // keys per tile

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Position (in 8-byte units) of the 4-key chunk c of V^T row d in LDS. Chunks
// are stored in pairs {4s + j, 4s + j + 2} (j = 0, 1), the two chunks one lane
// of the PV product reads, so they come back in one ds_read_b128. A 128-byte
// row covers half of the 64 LDS banks and a 16-byte read is served 16 lanes
// (16 consecutive rows) at a time, so pair slots are XOR-swizzled by d / 2:
// the 8 even and the 8 odd rows of a group each take 8 distinct slots
// (swizzling by d, rows d and d + 8 met in the same banks: counters showed a
// third of the LDS cycles stalled on bank conflicts).
__device__ __forceinline__ int vt_slot(int c, int d) {
  const int s4 = c >> 2, j = c & 3;              // c = 4*s4 + j
  const int pair = 2 * s4 + (j & 1);            // {4s+0, 4s+2} -> 2s, {4s+1, 4s+3} -> 2s+1
  const int half = j >> 1;                      // first or second chunk of the pair
  return (((pair ^ ((d >> 1) & 7)) << 1) | half);
}

// Row lookup of streaming mode: base of key row `p` (absolute position).
// Three sources: the chunk itself, the ring (sink slots, then the recent
// window), and a fixed chunk row for positions no query of the launch may
// attend (the mask removes them), so every address stays inside its buffer.
// All three are computed and one is selected, with no per-lane branch. A
// window position p (n - R <= p < n) has ring slot S + (p - S) mod R =
// S + (c0 + R + p - n) mod R with the uniform c0 = (n - S) mod R, and
// c0 + R + p - n lies in [c0, c0 + R): one conditional subtract instead of a
// per-lane division.
template <int D>
__device__ __forceinline__ const uint16_t* stream_row(const AttnArgs& a, int b, int kv, int p,
                                                      bool v) {
  const bool chunk = p >= a.n && p < a.n + a.T;
  const int rlo = a.n - a.R > a.S ? a.n - a.R : a.S;
  const bool ring = !chunk && p >= 0 && p < a.n && (p < a.S || p >= rlo);
  const int c0 = (int)((uint32_t)(a.n > a.S ? a.n - a.S : 0) % (uint32_t)a.R);
  const int q = c0 + a.R + (p - a.n);
  const int slot = p < a.S ? p : a.S + (q >= a.R ? q - a.R : q);
  const int64_t i_chunk = ((int64_t)b * a.T + (p - a.n)) * a.Hkv + kv;
  const int64_t i_ring = ((int64_t)b * a.Hs + (kv - a.Hr)) * (a.S + a.R) + slot;
  const int64_t i_mask = (int64_t)b * a.T * a.Hkv + kv;
  // both bases in scalar registers, so the per-lane choice is a register
  // select (not a load of the chosen pointer from the argument block)
  const uint16_t* ring_base = wave_ptr(v ? a.vr : a.kr);
  const uint16_t* in_base = wave_ptr(v ? a.v_in : a.k_in);
  return (ring ? ring_base : in_base) + (chunk ? i_chunk : ring ? i_ring : i_mask) * D;
}

// Waves per block: 8 (each staged K/V tile serves 256 query rows; waves 0-3
// stage V, waves 4-7 stage K).
template <int MODE>
constexpr int attn_waves() { return 8; }

template <int D, int HB, int MODE>
__global__ __launch_bounds__(64 * attn_waves<MODE>(), 1) void attn_kernel(AttnArgs a) {
  constexpr int NW = attn_waves<MODE>();
  constexpr int KS = D / 16;          // k-steps of the QK product
  constexpr int DB = D / 32;          // 32-row d-blocks of the PV product
  constexpr int TOKW = 32;            // tokens per wave
  constexpr int BMT = TOKW * NW / HB;  // tokens per block
  constexpr int KPAD = D + 8;         // K tile row stride in LDS (elements)
  constexpr int KLD = D / 32;         // 16-byte K loads per thread
  constexpr bool kMixed = MODE == MODE_MIXED || MODE == MODE_MIXED_BLOCK;
  constexpr bool kGrad = MODE == MODE_GRAD || MODE == MODE_GRAD_BLOCK;
  constexpr bool kBlock = MODE == MODE_MIXED_BLOCK || MODE == MODE_GRAD_BLOCK;
  // the gate-blended forward and its gate gradient visit the Lambda tiles,
  // then all causal tiles
  constexpr bool kTwoPhase = kMixed || kGrad;
  // two LDS stages: tile k is read from stage k & 1 while tile k + 1 is
  // written to the other, so one barrier per tile suffices
  __shared__ __align__(16) uint16_t Ks[2][kBN * KPAD];
  __shared__ __align__(16) uint16_t Vt[2][D * kBN];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int h2 = lane >> 5, q32 = lane & 31;
  const int b = blockIdx.z;
  const int groups = a.G / HB;
  // Blocks are dispatched in linear order, x fastest. With query tiles in y
  // the longest rows of every head come first (global longest-first order,
  // no late long blocks) and block i of a row lands on XCD i mod 8, so an XCD
  // sees only some heads' keys and values (L2 reuse).
  const int hg = (int)(a.tiles_in_y ? blockIdx.x : blockIdx.y);  // head group
  const int tq = (int)(a.tiles_in_y ? blockIdx.y : blockIdx.x);
  const int kv = a.kv_base + hg / groups;
  const int head = kv * a.G + (hg % groups) * HB + (wave % HB);
  const int tile = a.n_qtiles - 1 - tq;  // longest rows first
  const int tok0 = tile * BMT;
  const int t_q = tok0 + (wave / HB) * TOKW + q32;   // this lane's query token
  const int t_qc = t_q < a.T ? t_q : a.T - 1;
  const int i_q = a.n + t_q;                          // and its position
  const int blk_last = (tok0 + BMT < a.T ? tok0 + BMT : a.T) - 1;
  const int i_min = a.n + tok0, i_max = a.n + blk_last;
  // this wave's query positions (wave-uniform)
  const int w_tok0 = tok0 + (wave / HB) * TOKW;
  const int i_wfirst = a.n + w_tok0;
  const int i_wlast = a.n + (w_tok0 + TOKW - 1 < a.T ? w_tok0 + TOKW - 1 : a.T - 1);

  // ---- key tiles visited by this block --------------------------------------
  // Lambda tiles (the sink tiles, then the window tiles of the block's
  // queries) come first: they are the whole sequence in streaming mode and
  // phase 1 of the mixed forward; the causal tiles follow (retrieval mode,
  // phase 2 of the mixed forward).
  int n1 = 0, w0 = 0, nlam = 0, ntiles;
  // block-sparse Lambda (64-token blocks, the key tile): a key block is
  // visible when among the first sbk blocks or within rbk blocks of the
  // query's block
  constexpr bool lblk = kBlock;
  const int sbk = (a.S + kBN - 1) / kBN, rbk = (a.R + kBN - 1) / kBN;
  if constexpr (MODE != MODE_RETRIEVAL) {
    const int lo0 = lblk ? (i_min / kBN - rbk + 1) * kBN : i_min - a.R + 1;
    const int lo = lo0 > 0 ? lo0 : 0;
    const int s_eff = lblk ? sbk * kBN : a.S;
    const int sink_hi = s_eff < i_max + 1 ? s_eff : i_max + 1;
    n1 = (sink_hi + kBN - 1) / kBN;  // sink tiles cover [0, 64*n1)
    w0 = lo > kBN * n1 ? lo : kBN * n1;
    const int n2 = i_max >= w0 ? (i_max - w0) / kBN + 1 : 0;
    nlam = n1 + n2;
  }
  ntiles = MODE == MODE_STREAMING ? nlam : nlam + i_max / kBN + 1;
  auto tile_pos = [&](int k) {
    return k < nlam ? (k < n1 ? kBN * k : w0 + kBN * (k - n1)) : kBN * (k - nlam);
  };

  // ---- query fragments (B operand of S^T = K Q^T) ----------------------------
  bf16x8 qf[KS];
  {
    const uint16_t* qp = a.q + (((int64_t)b * a.T + t_qc) * a.Hq + head) * D + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(ld16(qp + 16 * ks));
  }

  // ---- global -> register staging of one K/V tile ------------------------------
  // 256 threads stage K and 256 stage V; the roles are wave-uniform.
  // Retrieval mode (the head's cached rows) and the mixed forward (the
  // sequence's rows of one KV head, a row stride of Hkv*D) read K and V each
  // as one buffer resource. Rows at or past the last key read as zeros (the
  // causal mask removes them), a tile's addresses are one add per lane (53
  // fewer VALU per tile than per-row pointers), and both roles load into one
  // set of registers (the 128-bit buffer loads keep their width; with plain
  // pointers a shared set made the compiler split them into 4-byte loads).
  // Streaming mode gathers rows per lane from the ring and the chunk and
  // keeps a set per role.
  static_assert(NW == 8, "the staging roles assume 8 waves");
  constexpr bool kBuf = MODE != MODE_STREAMING;
  const int st_t = tid & 255;
  const bool stage_k = wave >= 4;
  const int kr_row = st_t >> 2, kr_d0 = (st_t & 3) * (D / 4);
  const int vg = st_t & 15, vdc = st_t >> 4;  // V: keys 4vg..4vg+3, d-chunk 8*vdc
  const bool v_active = !stage_k && vdc < D / 8;
  u32x4 kreg[4];                    // K: KLD chunks of a row (and V when kBuf)
  u32x4 vown[kBuf ? 1 : 4];         // V: one d-chunk of 4 keys
  auto vreg = [&](int r) -> u32x4& {
    if constexpr (kBuf) return kreg[r];
    else return vown[r];
  };
  // buffer view: row stride, first element and readable bytes (the host
  // keeps every such range below 2^31 bytes)
  const uint32_t rstride = (uint32_t)(MODE == MODE_RETRIEVAL ? D * 2 : a.Hkv * D * 2);
  const int64_t hoff = MODE == MODE_RETRIEVAL ? ((int64_t)b * a.Hr + kv) * a.cap * D
                                              : ((int64_t)b * a.T * a.Hkv + kv) * D;
  const uint32_t rbytes =
      MODE == MODE_RETRIEVAL ? (uint32_t)(a.n + a.T) * (uint32_t)(D * 2)
                             : (uint32_t)((int64_t)a.T * a.Hkv - kv) * (uint32_t)(D * 2);
  const __amdgpu_buffer_rsrc_t krs =
      wave_rsrc((MODE == MODE_RETRIEVAL ? a.kc : a.k_in) + (kBuf ? hoff : 0), kBuf ? rbytes : 0u);
  const __amdgpu_buffer_rsrc_t vrs =
      wave_rsrc((MODE == MODE_RETRIEVAL ? a.vc : a.v_in) + (kBuf ? hoff : 0), kBuf ? rbytes : 0u);
  const uint32_t k_voff = (uint32_t)kr_row * rstride + (uint32_t)kr_d0 * 2u;
  const uint32_t v_voff = (uint32_t)(4 * vg) * rstride + (uint32_t)(8 * vdc) * 2u;
  auto load_k = [&](int p0) {
    if constexpr (kBuf) {
      const uint32_t o = k_voff + (uint32_t)p0 * rstride;
#pragma unroll
      for (int c = 0; c < KLD; ++c) kreg[c] = buf_ld16(krs, o + 16 * c, 0);
    } else {
      const uint16_t* kp = stream_row<D>(a, b, kv, p0 + kr_row, false) + kr_d0;
#pragma unroll
      for (int c = 0; c < KLD; ++c) kreg[c] = ld16(kp + 8 * c);
    }
  };
  auto load_v = [&](int p0) {
    if constexpr (kBuf) {
      const uint32_t o = v_voff + (uint32_t)p0 * rstride;
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg(r) = buf_ld16(vrs, o + (uint32_t)r * rstride, 0);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg(r) = ld16(stream_row<D>(a, b, kv, p0 + 4 * vg + r, true) + 8 * vdc);
    }
  };
  auto store_k = [&](int stage) {
    uint16_t* ks = Ks[stage];
#pragma unroll
    for (int c = 0; c < KLD; ++c) st16(ks + kr_row * KPAD + kr_d0 + 8 * c, kreg[c]);
  };
  auto store_v = [&](int stage) {
    uint16_t* vt = Vt[stage];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = 8 * vdc + i;
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      uint32_t lo = __builtin_amdgcn_perm(word_of(vreg(1), i >> 1), word_of(vreg(0), i >> 1), sel);
      uint32_t hi = __builtin_amdgcn_perm(word_of(vreg(3), i >> 1), word_of(vreg(2), i >> 1), sel);
      uint32_t* dst = reinterpret_cast<uint32_t*>(vt + d * kBN + 4 * vt_slot(vg, d));
      dst[0] = lo;
      dst[1] = hi;
    }
  };
  auto load_tile = [&](int p0) {
    if (stage_k) load_k(p0);
    if (v_active) load_v(p0);
  };
  auto store_tile = [&](int stage) {
    if (stage_k) store_k(stage);
    if (v_active) store_v(stage);
  };

  // ---- state --------------------------------------------------------------------
  // One softmax state (m, l, O). The mixed forward runs its Lambda phase in
  // it, folds (1 - alpha) * O / l into bf16 pairs and restarts it for the
  // causal phase, so it never holds two sets of accumulators. The folded
  // pairs are parked in LDS until the epilogue (each lane reads back only what
  // it wrote), which leaves the causal loop the registers the plain prefill
  // loop has (held in registers they made the compiler fetch the K fragments
  // two at a time, each pair of products waiting on its LDS read).
  f32x16 o_f[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o_f[db] = f32x16{};
  float m_f = -INFINITY, l_f = 0.0f;
  __shared__ uint32_t lam_lds[kMixed ? NW * DB * 8 * 64 : 1];
  auto lam_at = [&](int db, int i) -> uint32_t& {
    return lam_lds[((wave * DB + db) * 8 + i) * 64 + lane];
  };
  const float alpha = kMixed ? a.alpha[kv] : 1.0f;
  // Gate gradient: dout . (O / l) over this lane's channels of its query,
  // the element (db, 4 jb + r) of O being channel 32 db + 8 jb + 4 h2 + r.
  float g_lam = 0.0f;
  auto dout_dot = [&](float inv_l) -> float {
    const uint16_t* dp = a.dout + (((int64_t)b * a.T + t_qc) * a.Hq + head) * D + 4 * h2;
    float acc = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const uint2 w = *reinterpret_cast<const uint2*>(dp + 32 * db + 8 * jb);
        acc = fmaf(__uint_as_float(w.x << 16), o_f[db][4 * jb + 0], acc);
        acc = fmaf(__uint_as_float(w.x & 0xffff0000u), o_f[db][4 * jb + 1], acc);
        acc = fmaf(__uint_as_float(w.y << 16), o_f[db][4 * jb + 2], acc);
        acc = fmaf(__uint_as_float(w.y & 0xffff0000u), o_f[db][4 * jb + 3], acc);
      }
    return acc * inv_l;
  };

  // One online-softmax update of (m, l, O) from masked raw scores (m in raw
  // score units; the scale, folded with log2(e), enters the exp2 argument as
  // one FMA). m is a reference maximum, not necessarily the exact one: O and
  // l are rescaled only when some lane's tile maximum exceeds its m by more
  // than 8 in the log2 domain (wave-uniform test), so P stays at most 2^8 and
  // O / l is unchanged; most tiles skip the rescale. Returns P packed as the
  // B operands of the four 16-key slices.
  const float c2 = a.scale_log2;
  const float lazy = 8.0f / c2;  // raw-score growth that forces a rescale
  auto softmax_update = [&](const f32x16 (&sc)[2], float& m, float& l, f32x16 (&O)[DB],
                            bf16x8 (&pb)[4]) {
    float tm = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) tm = fmaxf(tm, sc[kb][j]);
    tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
    const float mn = fmaxf(m, tm);
    // m = -inf (no allowed key yet) and a finite tm always rescales
    if (__ballot(tm > m + lazy) != 0) {
      // m = -inf, mn finite -> 0; a lane still without an allowed key (both
      // -inf, l = 0 and O = 0) keeps factor 1 instead of exp2(NaN)
      const float corr = mn == -INFINITY ? 1.0f : fast_exp2((m - mn) * c2);
      l *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) O[db] *= corr;
      m = mn;
    }
    const float mc = m == -INFINITY ? 0.0f : m * c2;  // no allowed key yet: p = 0
    float p[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) p[kb][j] = fast_exp2(fmaf(sc[kb][j], c2, -mc));
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[s][i] = (__bf16)p[s >> 1][8 * (s & 1) + i];
    // the row sum adds the bf16 values the PV product uses, two per dot2
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 8; i += 4) {
        ls0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[s][i], pb[s][i + 1]}, ones, ls0, false);
        ls1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[s][i + 2], pb[s][i + 3]}, ones, ls1,
                                              false);
      }
    l += ls0 + ls1;
  };
  auto pv = [&](const uint16_t* vt, const bf16x8 (&pb)[4], f32x16 (&O)[DB]) {
    // all V^T fragments of two 16-key slices are requested before their
    // products (the empty asm keeps the compiler from sinking each read next
    // to its use, which would expose the LDS latency between products)
#pragma unroll
    for (int s2 = 0; s2 < 4; s2 += 2) {
      bf16x8 av[2][DB];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          // keys 16s+4h2..+3 and 16s+8+4h2..+3: one adjacent 16-byte pair
          const int d = 32 * db + q32;
          av[h][db] = as_bf16x8(
              *reinterpret_cast<const u32x4*>(vt + d * kBN + 4 * vt_slot(4 * (s2 + h) + h2, d)));
        }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[h][db], pb[s2 + h], O[db], 0, 0, 0);
    }
  };

  // S^T = K Q^T for the 64 keys of the K tile at ks (two 32-key blocks). All
  // K fragments of a block are requested before its first product (as for V
  // above), and the two blocks' independent accumulation chains are
  // interleaved.
  auto qk = [&](const uint16_t* ks, f32x16 (&st)[2]) {
    st[0] = f32x16{};
    st[1] = f32x16{};
    const uint16_t* krow0 = ks + q32 * KPAD + 8 * h2;
    const uint16_t* krow1 = krow0 + 32 * KPAD;
    bf16x8 ak0[KS], ak1[KS];
#pragma unroll
    for (int ks_ = 0; ks_ < KS; ++ks_)
      ak0[ks_] = as_bf16x8(*reinterpret_cast<const u32x4*>(krow0 + 16 * ks_));
    asm volatile("" ::: "memory");
#pragma unroll
    for (int ks_ = 0; ks_ < KS; ++ks_)
      ak1[ks_] = as_bf16x8(*reinterpret_cast<const u32x4*>(krow1 + 16 * ks_));
    asm volatile("" ::: "memory");
#pragma unroll
    for (int ks_ = 0; ks_ < KS; ++ks_) {
      st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak0[ks_], qf[ks_], st[0], 0, 0, 0);
      st[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak1[ks_], qf[ks_], st[1], 0, 0, 0);
    }
  };
  // Masked scores, softmax update and PV product of tile k from its raw
  // scores st and V tile vt. Tiles wholly below the wave's first query need
  // no causal mask, tiles wholly above its last query are skipped.
  auto consume = [&](int k, f32x16 (&st)[2], const uint16_t* vt) {
    const int p0 = tile_pos(k);
    const bool lam_phase = MODE == MODE_STREAMING || (kTwoPhase && k < nlam);
    const bool live = p0 <= i_wlast;
    const bool diag = p0 + kBN - 1 > i_wfirst;
    if (live) {
      // masked in place: unmasked tiles use the product registers as they are
      // (a separate masked copy cost 32 moves per tile on the unmasked path)
      if (lam_phase || diag) {
        // Element j of the lane's scores is key base + c_j, with c_j a
        // compile-time offset. One loop per mode (a tile-uniform branch
        // between two loops made the compiler copy the scores at the join
        // on every tile). Bitwise operators: a select per element, no
        // per-lane branches.
        const int base = p0 + 4 * h2;
        if constexpr (MODE == MODE_RETRIEVAL || lblk) {
          // causal: c_j <= dq; under the block mask a 64-key tile is one
          // block, visible to a query or not as a whole
          int dq = i_q - base;
          if constexpr (lblk) {
            const bool vis = ((p0 >> 6) < sbk) | (((i_q >> 6) - (p0 >> 6)) < rbk);
            dq = (lam_phase & !vis) ? -1 : dq;
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int c = 32 * kb + 8 * (j >> 2) + (j & 3);
              st[kb][j] = c <= dq ? st[kb][j] : -INFINITY;
            }
        } else {
          // token-level Lambda; outside the Lambda phase every key passes
          // the sink test, leaving the causal one
          const int s_lim = lam_phase ? a.S : 0x7fffffff;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int jp = base + 32 * kb + 8 * (j >> 2) + (j & 3);
              const bool ok = (jp <= i_q) & ((jp < s_lim) | (i_q - jp < a.R));
              st[kb][j] = ok ? st[kb][j] : -INFINITY;
            }
        }
      }
      bf16x8 pb[4];
      softmax_update(st, m_f, l_f, o_f, pb);
      pv(vt, pb, o_f);
    }
  };

  // ---- main loop ----------------------------------------------------------------
  {
    load_tile(tile_pos(0));
    store_tile(0);
    __syncthreads();
    // Every load issued so far (the query fragments, tile 0) has landed: say
    // so explicitly. Without it the wait-count insertion merges the path on
    // which no tile store waited into the loop header and keeps the query
    // loads "pending", so each iteration's QK products would wait for the
    // next tile's prefetch (vmcnt counts in order), exposing its whole
    // latency.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    for (int k = 0; k < ntiles; ++k) {
      const int stage = k & 1;
      const bool more = k + 1 < ntiles;
      if (more) load_tile(tile_pos(k + 1));
      if (kTwoPhase && k == nlam) {
        // end of the Lambda phase: keep (1 - alpha) * O / l (forward) or
        // dout . O / l (gate gradient), restart the state
        const float ll = l_f + __shfl_xor(l_f, 32, 64);
        if constexpr (kGrad) {
          g_lam = dout_dot(1.0f / ll);
        } else {
          const float wl = (1.0f - alpha) / ll;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 8; ++i)
              lam_at(db, i) = pack_bf16x2(o_f[db][2 * i] * wl, o_f[db][2 * i + 1] * wl);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) o_f[db] = f32x16{};
        m_f = -INFINITY;
        l_f = 0.0f;
      }
      f32x16 st[2];
      qk(Ks[stage], st);
      consume(k, st, Vt[stage]);
      // the other stage was last read before the previous barrier
      if (more) store_tile(stage ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue -----------------------------------------------------------------
  if constexpr (kGrad) {
    // dout . (full - streaming) summed over the block's rows and channels
    // (all waves belong to one KV head); one partial per block, summed per
    // KV head by the reduction kernel in a fixed order
    const float lf = l_f + __shfl_xor(l_f, 32, 64);
    float g = t_q < a.T ? dout_dot(1.0f / lf) - g_lam : 0.0f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) g += __shfl_xor(g, off, 64);
    __shared__ float gsum[NW];
    if (lane == 0) gsum[wave] = g;
    __syncthreads();
    if (threadIdx.x == 0) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += gsum[w];
      a.partial[((int64_t)b * a.Hkv * groups + hg) * a.n_qtiles + tq] = sum;
    }
    return;
  }
  if (t_q >= a.T) return;
  const float lf = l_f + __shfl_xor(l_f, 32, 64);
  const float wf = alpha / lf;  // alpha = 1 outside the mixed forward
  uint16_t* op = a.out + (((int64_t)b * a.T + t_q) * a.Hq + head) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = o_f[db][4 * jb + r] * wf;
        if constexpr (kMixed) {
          const uint32_t w = lam_at(db, (4 * jb + r) >> 1);
          v[r] += __uint_as_float((r & 1) ? (w & 0xffff0000u) : (w << 16));
        }
      }
      uint2 w;
      w.x = pack_bf16x2(v[0], v[1]);
      w.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(op + 32 * db + 8 * jb + 4 * h2) = w;
    }
}

// ---- launchers -------------------------------------------------------------------
template <int D, int HB, int MODE>
static hipError_t launch_hb(const AttnArgs& a, int n_kv, int B, hipStream_t s) {
  constexpr int NW = attn_waves<MODE>();
  constexpr int BMT = 32 * NW / HB;
  AttnArgs x = a;
  x.n_qtiles = (a.T + BMT - 1) / BMT;
  const unsigned hgs = (unsigned)(n_kv * (a.G / HB));
  // Long rows (retrieval, mixed) launch longest-first across all heads with
  // the query tiles in y. Streaming blocks visit a few tiles each and are
  // alike, so the order's gain is absent while neighbouring blocks on
  // different heads lose the L2 reuse of one head's ring and chunk rows: query
  // tiles in x ran 42 instead of 59 us per 8192-token chunk of the Llama-3-8B
  // layer. The y extent of a grid is 16 bits.
  x.tiles_in_y = MODE != MODE_STREAMING && x.n_qtiles <= 65535;
  dim3 grid(x.tiles_in_y ? hgs : (unsigned)x.n_qtiles, x.tiles_in_y ? (unsigned)x.n_qtiles : hgs,
            (unsigned)B);
  attn_kernel<D, HB, MODE><<<grid, 64 * NW, 0, s>>>(x);
  return hipGetLastError();
}

template <int D, int MODE>
static hipError_t launch_d(const AttnArgs& a, int n_kv, int B, hipStream_t s) {
  switch (a.G) {
    case 1: return launch_hb<D, 1, MODE>(a, n_kv, B, s);
    case 2: return launch_hb<D, 2, MODE>(a, n_kv, B, s);
    default: return launch_hb<D, 4, MODE>(a, n_kv, B, s);  // G = 4 or 8
  }
}

template <int MODE>
static hipError_t launch_mode(const AttnArgs& a, int D, int n_kv, int B, hipStream_t s) {
  if (n_kv <= 0 || a.T <= 0) return hipSuccess;
  return D == 128 ? launch_d<128, MODE>(a, n_kv, B, s) : launch_d<64, MODE>(a, n_kv, B, s);
}

static AttnArgs base_args(const duo_layer* L, const void* q, int T, void* out) {
  const duo_layer_desc& d = L->d;
  AttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.out = static_cast<uint16_t*>(out);
  a.T = T;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.Hr = L->Hr;
  a.Hs = L->Hs;
  a.G = L->G;
  a.S = d.sink;
  a.R = d.recent;
  a.cap = d.retrieval_capacity;
  a.n = (int)L->n;
  a.scale_log2 = d.softmax_scale * kLog2e;
  a.kc = reinterpret_cast<const uint16_t*>(L->rbuf + L->lay.k_offset);
  a.vc = reinterpret_cast<const uint16_t*>(L->rbuf + L->lay.v_offset);
  a.kr = reinterpret_cast<const uint16_t*>(L->sbuf + L->lay.ring_k_offset);
  a.vr = reinterpret_cast<const uint16_t*>(L->sbuf + L->lay.ring_v_offset);
  return a;
}

hipError_t launch_prefill_retrieval(const duo_layer* L, const void* q, int T, void* out,
                                    hipStream_t s) {
  AttnArgs a = base_args(L, q, T, out);
  a.kv_base = 0;
  return launch_mode<MODE_RETRIEVAL>(a, L->d.head_dim, L->Hr, L->d.batch, s);
}

hipError_t launch_prefill_streaming(const duo_layer* L, const void* q, const void* k,
                                    const void* v, int T, void* out, hipStream_t s) {
  AttnArgs a = base_args(L, q, T, out);
  a.k_in = static_cast<const uint16_t*>(k);
  a.v_in = static_cast<const uint16_t*>(v);
  a.kv_base = L->Hr;
  return launch_mode<MODE_STREAMING>(a, L->d.head_dim, L->Hs, L->d.batch, s);
}

hipError_t launch_mixed(const duo_layer_desc& d, const void* q, const void* k, const void* v,
                        const float* alpha, int T, int lam_block, void* out, hipStream_t s) {
  AttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.out = static_cast<uint16_t*>(out);
  a.k_in = static_cast<const uint16_t*>(k);
  a.v_in = static_cast<const uint16_t*>(v);
  a.alpha = alpha;
  a.T = T;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.G = d.n_q_heads / d.n_kv_heads;
  a.S = d.sink;
  a.R = d.recent;
  a.n = 0;
  a.kv_base = 0;
  a.scale_log2 = d.softmax_scale * kLog2e;
  return lam_block ? launch_mode<MODE_MIXED_BLOCK>(a, d.head_dim, d.n_kv_heads, d.batch, s)
                   : launch_mode<MODE_MIXED>(a, d.head_dim, d.n_kv_heads, d.batch, s);
}

// Gate gradient: the flash pass writes one partial sum per block; this
// kernel adds a KV head's partials in a fixed order (one block per KV head)
// and the L1 term's gradient l1 * sign(alpha), taken as 0 at alpha = 0.
__global__ __launch_bounds__(256) void alpha_grad_reduce_kernel(const float* __restrict__ partial,
                                                                int B, int Hkv, int per_kv,
                                                                const float* __restrict__ alpha,
                                                                float l1, float* __restrict__ grad) {
  __shared__ float red[256];
  const int kv = blockIdx.x;
  float s = 0.0f;
  const int n = B * per_kv;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int bb = i / per_kv, j = i - bb * per_kv;
    s += partial[((int64_t)bb * Hkv + kv) * per_kv + j];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float al = alpha[kv];
    grad[kv] = red[0] + l1 * (al > 0.0f ? 1.0f : (al < 0.0f ? -1.0f : 0.0f));
  }
}

// Heads per block of the flash kernels for group size G (as launch_d picks).
static int heads_per_block(int G) { return G == 1 ? 1 : (G == 2 ? 2 : 4); }

size_t mixed_grad_partials(const duo_layer_desc& d, int T) {
  const int G = d.n_q_heads / d.n_kv_heads, HB = heads_per_block(G);
  const int BMT = 32 * 8 / HB;
  return (size_t)d.batch * d.n_kv_heads * (G / HB) * (size_t)((T + BMT - 1) / BMT);
}

hipError_t launch_mixed_alpha_grad(const duo_layer_desc& d, const void* q, const void* k,
                                   const void* v, const void* dout, const float* alpha,
                                   float l1_weight, int T, int lam_block, float* grad,
                                   float* partial, hipStream_t s) {
  AttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.k_in = static_cast<const uint16_t*>(k);
  a.v_in = static_cast<const uint16_t*>(v);
  a.dout = static_cast<const uint16_t*>(dout);
  a.partial = partial;
  a.alpha = alpha;
  a.T = T;
  a.Hq = d.n_q_heads;
  a.Hkv = d.n_kv_heads;
  a.G = d.n_q_heads / d.n_kv_heads;
  a.S = d.sink;
  a.R = d.recent;
  a.n = 0;
  a.kv_base = 0;
  a.scale_log2 = d.softmax_scale * kLog2e;
  hipError_t e = lam_block
                     ? launch_mode<MODE_GRAD_BLOCK>(a, d.head_dim, d.n_kv_heads, d.batch, s)
                     : launch_mode<MODE_GRAD>(a, d.head_dim, d.n_kv_heads, d.batch, s);
  if (e != hipSuccess) return e;
  const int HB = heads_per_block(a.G), BMT = 32 * 8 / HB;
  const int per_kv = (a.G / HB) * ((T + BMT - 1) / BMT);
  alpha_grad_reduce_kernel<<<d.n_kv_heads, 256, 0, s>>>(partial, d.batch, d.n_kv_heads, per_kv,
                                                        alpha, l1_weight, grad);
  return hipGetLastError();
}

}  // namespace duo
