// Tiled softmax attention on MFMA (bf16, or fp16 for fp16 and 4-bit caches)
// for the prefill paths and the gate-blended identification forward.
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
//     K/V tile in LDS serves 8 waves of query rows;
//   * the mixed forward runs in two phases over one tile pipeline and one
//     softmax state: the Lambda tiles (sinks and the window band, a few per
//     query tile) first, folded into (1 - alpha) * O / l kept as bf16 pairs,
//     then all causal tiles as in retrieval mode (the band's QK products are
//     computed twice; two sets of accumulators would halve the occupancy);
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 (the f16
//     form for fp16 and 4-bit caches). In this
//     orientation a lane holds one query's scores, so the softmax needs one
//     cross-lane exchange per tile, and the score accumulator is directly the
//     B operand of the PV product (keys permuted inside each 16-key slice,
//     which a sum over keys does not see);
//   * K and V tiles go from global memory straight into LDS (16-byte buffer
//     loads with the LDS bit: no VGPRs, no repacking VALU, no ds_write), all
//     8 waves issuing a share. Both are stored row-major with 16-byte chunks
//     XOR-swizzled by row. K fragments are one ds_read_b128 each; V^T
//     fragments are two transposed reads (ds_read_b64_tr_b16) each, so V
//     needs no transposing copy. Streaming mode, which gathers rows from the
//     ring and the chunk per lane, and the 4-bit mode, which decodes codes,
//     stage through registers instead (K rows padded by 16 bytes, V
//     transposed on the way to LDS);
//   * the next tile's loads are in flight while the current tile is
//     computed; query tiles are launched longest-first (causal imbalance);
//   * output rows leave through LDS as whole rows (coalesced stores).
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "duo_internal.hpp"
#include "mfma_common.hpp"

namespace duo {

// Kernel modes; the _BLOCK variants take the streaming part of the
// two-phase modes under the block-sparse Lambda mask.
enum {
  MODE_RETRIEVAL = 0,
  MODE_STREAMING = 1,
  MODE_MIXED = 2,
  MODE_GRAD = 3,
  MODE_MIXED_BLOCK = 4,
  MODE_GRAD_BLOCK = 5,
  // fp16 forms of the prefill (layers with an fp16 or 4-bit cache): K/V tiles,
  // P and the products in fp16; the 4-bit form dequantises its tiles on the
  // way to LDS
  MODE_RETRIEVAL_I4 = 6,
  MODE_RETRIEVAL_F16 = 7,
  MODE_STREAMING_F16 = 8
};
constexpr bool mode_f16(int m) {
  return m == MODE_RETRIEVAL_I4 || m == MODE_RETRIEVAL_F16 || m == MODE_STREAMING_F16;
}
constexpr bool mode_streaming(int m) { return m == MODE_STREAMING || m == MODE_STREAMING_F16; }
// causal attention of a chunk over the retrieval cache
constexpr bool mode_cache(int m) {
  return m == MODE_RETRIEVAL || m == MODE_RETRIEVAL_F16 || m == MODE_RETRIEVAL_I4;
}

struct AttnArgs {
  const uint16_t* q;     // [B][T][Hq][D]
  uint16_t* out;         // [B][T][Hq][D]
  const uint16_t* k_in;  // chunk / sequence K, V [B][T][Hkv][D]
  const uint16_t* v_in;
  const uint16_t* kc;    // retrieval cache [B][Hr][cap][D]
  const uint16_t* vc;
  const uint16_t* kr;    // ring [B][Hs][S+R][D]
  const uint16_t* vr;
  const uint8_t* kcodes;   // 4-bit retrieval cache (MODE_RETRIEVAL_I4): [B][Hr][cap32][D/2]
  const uint8_t* vcodes;   // [B][Hr][cap32/32][16 D] in the decode's PV operand order
  const uint32_t* ksz;     // [B][Hr][cap32/32][D/32][32] fp16 scale | fp16 zero << 16
  const uint32_t* vsz;
  int64_t cap32;
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

// Row lookup of streaming mode for a tile that starts inside the chunk: the
// chunk's row, positions past its end clamped to its last row (masked: a key
// after every query of the launch).
template <int D>
__device__ __forceinline__ const uint16_t* chunk_row(const AttnArgs& a, int b, int kv, int p,
                                                     bool v) {
  const int last = a.n + a.T - 1;
  const int t = (p < last ? p : last) - a.n;
  return wave_ptr(v ? a.v_in : a.k_in) + (((int64_t)b * a.T + t) * a.Hkv + kv) * D;
}

// Waves per block: 8 (each staged K/V tile serves 256 query rows; with
// register staging waves 0-3 stage V and waves 4-7 K, with direct loads every
// wave issues a share of both).
template <int MODE>
constexpr int attn_waves() { return 8; }

// Modes that can keep the softmax reference inside the QK product (q scaled
// by scale * log2(e) and rounded once to the operand type); the others
// always apply the scale in fp32.
constexpr bool mode_prescale(int m) {
  return m == MODE_RETRIEVAL || m == MODE_RETRIEVAL_F16 || m == MODE_MIXED ||
         m == MODE_MIXED_BLOCK || m == MODE_GRAD || m == MODE_GRAD_BLOCK;
}

// PRE: the pre-scaled form above where the mode has it; false applies the
// scale in fp32 (one FMA per score), exact for logits of any size.
template <int D, int HB, int MODE, bool PRE>
__device__ __forceinline__ void attn_body(AttnArgs a) {
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
  constexpr bool kStream = mode_streaming(MODE);
  constexpr bool kCache = mode_cache(MODE);
  constexpr bool kI4 = MODE == MODE_RETRIEVAL_I4;
  constexpr bool kF16 = mode_f16(MODE);
  using E8 = elem8<kF16>;  // MFMA operand: 8 bf16 or 8 fp16 values
  using Elem = std::conditional_t<kF16, _Float16, __bf16>;
  using E2 = std::conditional_t<kF16, f16x2, bf16x2>;
  // the gate-blended forward and its gate gradient visit the Lambda tiles,
  // then all causal tiles
  constexpr bool kTwoPhase = kMixed || kGrad;
  // Modes that read K and V through one buffer resource each stage them
  // with direct global->LDS loads (see below); streaming mode gathers rows
  // per lane, and the 4-bit mode dequantises codes, through registers.
  constexpr bool kDma = !kStream && !kI4;
  // Retrieval modes over 16-bit caches keep the softmax reference in the
  // product itself: q is scaled by scale * log2(e) once per block and each
  // QK accumulation starts from a register block holding -m, so a product
  // already is the exp2 argument (no FMA per score). The other modes stay
  // with raw scores: the streaming form has no 16 registers to spare, the
  // 4-bit form few.
  constexpr bool kRel = PRE && mode_prescale(MODE);
  constexpr int KROW = kDma ? D : KPAD;  // K tile row stride in LDS (elements)
  // two LDS stages: tile k is read from stage k & 1 while tile k + 1 is
  // written to the other, so one barrier per tile suffices. The stages are
  // separate arrays, each named statically in the (twice unrolled) loop, so
  // the compiler sees that reads of one stage do not wait for the direct
  // loads into the other.
  // (32-byte alignment: LDS variables are laid out by alignment, then size,
  // so the stages come before the gate-blended forward's 64 KB parking array
  // and stay below 64 KB, where a read's 16-bit immediate offset reaches them;
  // above it every operand address took a v_add)
  __shared__ __align__(32) uint16_t Ks0[kBN * KROW];
  __shared__ __align__(32) uint16_t Ks1[kBN * KROW];
  __shared__ __align__(32) uint16_t Vs0[D * kBN];
  __shared__ __align__(32) uint16_t Vs1[D * kBN];

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
  if constexpr (!kCache) {
    const int lo0 = lblk ? (i_min / kBN - rbk + 1) * kBN : i_min - a.R + 1;
    const int lo = lo0 > 0 ? lo0 : 0;
    const int s_eff = lblk ? sbk * kBN : a.S;
    const int sink_hi = s_eff < i_max + 1 ? s_eff : i_max + 1;
    n1 = (sink_hi + kBN - 1) / kBN;  // sink tiles cover [0, 64*n1)
    w0 = lo > kBN * n1 ? lo : kBN * n1;
    const int n2 = i_max >= w0 ? (i_max - w0) / kBN + 1 : 0;
    nlam = n1 + n2;
  }
  ntiles = kStream ? nlam : nlam + i_max / kBN + 1;
  auto tile_pos = [&](int k) {
    return k < nlam ? (k < n1 ? kBN * k : w0 + kBN * (k - n1)) : kBN * (k - nlam);
  };

  // ---- query fragments (B operand of S^T = K Q^T) ----------------------------
  E8 qf[KS];
  {
    const uint16_t* qp = a.q + (((int64_t)b * a.T + t_qc) * a.Hq + head) * D + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 w = ld16(qp + 16 * ks);
      if constexpr (kF16) {
        // bf16 -> fp32 (exact) -> fp16 (exact for magnitudes in fp16's normal
        // range: a bf16 significand has 8 bits, fp16's 11)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t wi = word_of(w, i >> 1);
          qf[ks][i] = (_Float16)__uint_as_float((i & 1) ? (wi & 0xffff0000u) : (wi << 16));
        }
      } else {
        qf[ks] = as_bf16x8(w);
      }
      if constexpr (kRel) {
        // q * scale * log2(e), rounded once to the operand type
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[ks][i] = (Elem)((float)qf[ks][i] * a.scale_log2);
      }
    }
  }

  // ---- staging of one K/V tile ---------------------------------------------------
  static_assert(NW == 8, "the staging roles assume 8 waves");
  // Buffer view of K and V: row stride, first element and readable bytes
  // (the host keeps every such range below 2^31 bytes). Retrieval mode reads
  // the head's cached rows, the mixed forward the sequence's rows of one KV
  // head (a row stride of Hkv*D).
  const uint32_t rstride = (uint32_t)(kCache ? D * 2 : a.Hkv * D * 2);
  const int64_t hoff = kCache ? ((int64_t)b * a.Hr + kv) * a.cap * D
                              : ((int64_t)b * a.T * a.Hkv + kv) * D;
  const uint32_t rbytes = kCache ? (uint32_t)(a.n + a.T) * (uint32_t)(D * 2)
                                 : (uint32_t)((int64_t)a.T * a.Hkv - kv) * (uint32_t)(D * 2);
  const __amdgpu_buffer_rsrc_t krs =
      wave_rsrc((kCache ? a.kc : a.k_in) + (kDma ? hoff : 0), kDma ? rbytes : 0u);
  const __amdgpu_buffer_rsrc_t vrs =
      wave_rsrc((kCache ? a.vc : a.v_in) + (kDma ? hoff : 0), kDma ? rbytes : 0u);

  // Direct loads (kDma). A 16-byte buffer load with the LDS bit writes lane
  // i's data to the instruction's LDS base + 16 i, so a 1 KB block of a tile
  // is filled by giving each lane the source chunk that belongs in its slot.
  // Rows are 2D bytes, unpadded, with 16-byte chunks XOR-swizzled by row so
  // that the MFMA operand reads below spread over the LDS banks:
  //   K: chunk c of row r sits in slot c ^ ksw(r), ksw(r) = r & 15 for
  //      256-byte rows and (r >> 1) & 7 for 128-byte rows: the 16 rows that
  //      16 lanes read together take 16 distinct slots of a 256-byte window;
  //   V: 32-byte segment g of row r sits in segment g ^ vsw(r), vsw(r) =
  //      2 (r & 3) for 256-byte rows and r & 3 for 128-byte rows: a
  //      transposed read takes 4 consecutive rows x 2 adjacent segments per
  //      32 lanes, 8 distinct segments.
  // Each wave issues D/64 loads of K and D/64 of V per tile. Rows past the
  // last key are clamped to it: the mask removes them, their values only
  // have to be finite. Neither the data nor its repacking passes through
  // VGPRs.
  constexpr int RB = 2 * D;       // bytes per LDS row (direct layout)
  constexpr int SPR = RB / 16;    // 16-byte slots per row
  constexpr int RPI = 64 / SPR;   // rows per 1 KB load
  constexpr int NIW = D / 64;     // loads per wave per tensor and tile
  // the swizzles, the XOR addressing of the operand reads and the 8 x NIW
  // loads covering a 64-row tile hold for these row sizes only
  static_assert(D == 64 || D == 128, "direct-load layout: 128- or 256-byte rows");
  static_assert(8 * NIW * RPI == kBN, "the block's loads cover one tile");
  auto ksw = [](int r) { return RB == 256 ? (r & 15) : ((r >> 1) & 7); };
  auto vsw = [](int r) { return RB == 256 ? 2 * (r & 3) : (r & 3); };
  const int last_row = (kCache ? a.n + a.T : a.T) - 1;
  const int dma_row0 = wave * NIW * RPI + lane / SPR;  // this lane's row in the wave's first block
  uint32_t k_c16[NIW], v_c16[NIW];  // byte offset of the chunk a lane fetches within its row
  uint32_t k_lo[NIW], v_lo[NIW];    // and of that chunk within the tile (row offset added)
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int r = dma_row0 + j * RPI, pos = lane % SPR;
    k_c16[j] = (uint32_t)(pos ^ ksw(r)) * 16u;
    v_c16[j] = (uint32_t)(2 * ((pos >> 1) ^ vsw(r)) + (pos & 1)) * 16u;
    k_lo[j] = (uint32_t)r * rstride + k_c16[j];
    v_lo[j] = (uint32_t)r * rstride + v_c16[j];
  }
  // the rows p0 .. p0 + 63 of one tensor into the stage at dst. A tile
  // wholly before the last key takes its row offset as the scalar offset and
  // the lane's offset within the tile from a register (no address VALU per
  // tile); the last tile clamps each lane's row to the last key.
  auto dma_rows = [&](int p0, uint16_t* dst, __amdgpu_buffer_rsrc_t rs,
                      const uint32_t (&c16)[NIW], const uint32_t (&lo)[NIW]) {
    if (p0 + kBN - 1 <= last_row) {
      const uint32_t so = (uint32_t)p0 * rstride;  // wave-uniform
#pragma unroll
      for (int j = 0; j < NIW; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(dst + (wave * NIW + j) * 512), 16,
                                                 (int)lo[j], (int)so, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < NIW; ++j) {
        const int blk = wave * NIW + j;  // the wave's j-th 1 KB block of the tile
        int r = p0 + dma_row0 + j * RPI;
        r = r < last_row ? r : last_row;
        const uint32_t ro = (uint32_t)r * rstride;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(dst + blk * 512), 16,
                                                 (int)(ro + c16[j]), 0, 0, 0);
      }
    }
  };

  // Register staging (streaming mode): 256 threads gather K rows and 256
  // threads V rows per lane from the ring and the chunk; V is transposed
  // into d-major rows (vt_slot) on the way to LDS.
  const int st_t = tid & 255;
  const bool stage_k = wave >= 4;
  const int kr_row = st_t >> 2, kr_d0 = (st_t & 3) * (D / 4);
  const int vg = st_t & 15, vdc = st_t >> 4;  // V: keys 4vg..4vg+3, d-chunk 8*vdc
  const bool v_active = !stage_k && vdc < D / 8;
  u32x4 kreg[4];  // K: KLD chunks of a row (unused, and removed, in the direct modes)
  u32x4 vown[4];  // V: one d-chunk of 4 keys
  // (tiles that start inside the chunk, p0 >= n, a wave-uniform test, read
  // chunk rows only)
  auto load_k = [&](int p0) {
    const uint16_t* kp;
    if (p0 >= a.n)
      kp = chunk_row<D>(a, b, kv, p0 + kr_row, false) + kr_d0;
    else
      kp = stream_row<D>(a, b, kv, p0 + kr_row, false) + kr_d0;
#pragma unroll
    for (int c = 0; c < KLD; ++c) kreg[c] = ld16(kp + 8 * c);
  };
  auto load_v = [&](int p0) {
    if (p0 >= a.n) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vown[r] = ld16(chunk_row<D>(a, b, kv, p0 + 4 * vg + r, true) + 8 * vdc);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vown[r] = ld16(stream_row<D>(a, b, kv, p0 + 4 * vg + r, true) + 8 * vdc);
    }
  };
  auto store_k = [&](uint16_t* ks) {
#pragma unroll
    for (int c = 0; c < KLD; ++c) st16(ks + kr_row * KPAD + kr_d0 + 8 * c, kreg[c]);
  };
  auto store_v = [&](uint16_t* vt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = 8 * vdc + i;
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      uint32_t lo = __builtin_amdgcn_perm(word_of(vown[1], i >> 1), word_of(vown[0], i >> 1), sel);
      uint32_t hi = __builtin_amdgcn_perm(word_of(vown[3], i >> 1), word_of(vown[2], i >> 1), sel);
      uint32_t* dst = reinterpret_cast<uint32_t*>(vt + d * kBN + 4 * vt_slot(vg, d));
      dst[0] = lo;
      dst[1] = hi;
    }
  };

  // 4-bit staging (retrieval heads of a 4-bit cache). The codes and the
  // scale/zero words are loaded before the current tile's products and
  // decoded as fma(code, scale, zero) in fp32, rounded to fp16, after them.
  //   K: thread (row, quarter) takes the D/4 channels kr_d0 .. of key row
  //      kr_row (D/8 code bytes, one group's scale/zero word), written to the
  //      padded row layout above.
  //   V: in a 32-token block the 16-byte code unit u = 4 (16 ch + cl) + mh
  //      holds channels 64 ch + 16 cq + cl (cq = 0..3, byte 4 cq + i) of
  //      tokens 4 mh + i (low nibbles) and 16 + 4 mh + i (high nibbles); a
  //      tile is two blocks, D units each, one unit per thread. Its 4 x 8
  //      values become eight 4-key chunks of V^T rows (vt_slot).
  // Rows past the last key: K rows are clamped to it (finite, masked); V
  // values are set to zero (the scale/zero words of unwritten rows are not
  // data), blocks past the last one clamped to it so every read stays inside
  // the head's arrays.
  const int64_t bh = (int64_t)b * a.Hr + kv;
  const int nblk32 = (int)(a.cap32 >> 5);
  const int vi_b2 = st_t / D, vi_u = st_t % D;  // V: block of the tile, code unit
  const int vi_mh = vi_u & 3, vi_cl = (vi_u >> 2) & 15, vi_ch = vi_u >> 6;
  const bool vi_active = !stage_k && st_t < 2 * D;
  constexpr int KCW = D / 32;  // code words (8 channels each) of a K thread
  uint32_t kcode[KCW], kszw = 0;
  u32x4 vcode = {}, vszq[4] = {};
  auto load_k_i4 = [&](int p0) {
    int r = p0 + kr_row;
    r = r < last_row ? r : last_row;
    const uint32_t* cp =
        reinterpret_cast<const uint32_t*>(a.kcodes + (bh * a.cap32 + r) * (D / 2) + kr_d0 / 2);
#pragma unroll
    for (int i = 0; i < KCW; ++i) kcode[i] = cp[i];
    kszw = a.ksz[((bh * nblk32 + (r >> 5)) * (D / 32) + kr_d0 / 32) * 32 + (r & 31)];
  };
  auto store_k_i4 = [&](uint16_t* ks) __attribute__((always_inline)) {
    const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(kszw & 0xffffu));
    const float zp = (float)__builtin_bit_cast(_Float16, (uint16_t)(kszw >> 16));
#pragma unroll
    for (int i = 0; i < KCW; ++i) {
      // byte j of word i: channels 8 i + 2 j (low nibble) and 8 i + 2 j + 1
      const uint32_t lo = kcode[i] & 0x0f0f0f0fu, hi = (kcode[i] >> 4) & 0x0f0f0f0fu;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2 h = {(_Float16)fmaf((float)((lo >> (8 * j)) & 0xffu), sc, zp),
                         (_Float16)fmaf((float)((hi >> (8 * j)) & 0xffu), sc, zp)};
        w[j] = __builtin_bit_cast(uint32_t, h);
      }
      st16(ks + kr_row * KPAD + kr_d0 + 8 * i, u32x4{w[0], w[1], w[2], w[3]});
    }
  };
  auto load_v_i4 = [&](int p0) {
    int blk = (p0 >> 5) + vi_b2;
    blk = blk < (last_row >> 5) ? blk : (last_row >> 5);
    const int64_t bb = bh * nblk32 + blk;
    vcode = ld16(a.vcodes + bb * (16 * D) + 16 * vi_u);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int run = 0; run < 2; ++run)
        vszq[2 * gi + run] =
            ld16(a.vsz + (bb * (D / 32) + 2 * vi_ch + gi) * 32 + 16 * run + 4 * vi_mh);
  };
  auto store_v_i4 = [&](uint16_t* vt, int p0) __attribute__((always_inline)) {
    const int tok0 = p0 + 32 * vi_b2 + 4 * vi_mh;  // token of run 0, i = 0
#pragma unroll
    for (int cq = 0; cq < 4; ++cq) {
      const int d = 64 * vi_ch + 16 * cq + vi_cl;
      const uint32_t cw = word_of(vcode, cq);
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const uint32_t nib = run ? (cw >> 4) & 0x0f0f0f0fu : cw & 0x0f0f0f0fu;
        const u32x4& sz = vszq[2 * (cq >> 1) + run];
        _Float16 x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = tok0 + 16 * run + i <= last_row;
          const uint32_t w = ok ? word_of(sz, i) : 0u;  // scale = zero = 0: value 0
          x[i] = (_Float16)fmaf((float)((nib >> (8 * i)) & 0xffu),
                                (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)),
                                (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)));
        }
        const int c4 = 8 * vi_b2 + 4 * run + vi_mh;  // 4-key chunk of the tile
        uint2 o;
        o.x = __builtin_bit_cast(uint32_t, f16x2{x[0], x[1]});
        o.y = __builtin_bit_cast(uint32_t, f16x2{x[2], x[3]});
        *reinterpret_cast<uint2*>(vt + d * kBN + 4 * vt_slot(c4, d)) = o;
      }
    }
  };

  int staged_p0 = 0;  // position of the tile held in the staging registers
  auto load_tile = [&](int p0) {
    if constexpr (kI4) {
      staged_p0 = p0;
      if (stage_k) load_k_i4(p0);
      if (vi_active) load_v_i4(p0);
    } else {
      if (stage_k) load_k(p0);
      if (v_active) load_v(p0);
    }
  };
  // (always_inline: the compiler outlined the 4-bit form, moving every
  // captured staging register to scratch memory)
  auto store_tile = [&](uint16_t* ks, uint16_t* vt) __attribute__((always_inline)) {
    if constexpr (kI4) {
      if (stage_k) store_k_i4(ks);
      if (vi_active) store_v_i4(vt, staged_p0);
    } else {
      if (stage_k) store_k(ks);
      if (v_active) store_v(vt);
    }
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
  float mc_f = 0.0f;  // m_f * scale_log2, or 0 while m_f = -inf (no allowed key yet)
  // kRel: mc_f is the reference in exp2 units (0 while the lane has seen no
  // allowed key, unset), and neg_m holds -mc_f in each of its 16 elements:
  // the QK accumulators start from it. Kept opaque so the compiler holds the
  // block in registers rather than rebuilding it from mc_f on every tile.
  bool unset = true;
  f32x16 neg_m{};
  if constexpr (kRel) asm volatile("" : "+v"(neg_m));
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
  auto softmax_rescale = [&](const f32x16 (&sc)[2], float& m, float& mc, float& l,
                             f32x16 (&O)[DB]) {
    float tm = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) tm = fmaxf(tm, sc[kb][j]);
    {
      // lanes l and l + 32 hold the two halves of a query's keys: one
      // v_permlane32_swap gives every lane its partner's maximum
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm), __float_as_uint(tm),
                                                       false, false);
      // one v_max_f32 of the pair (scores are never NaN, so the two
      // quieting maxima the compiler puts around values it did not produce
      // itself are not needed)
      asm("v_max_f32 %0, %1, %2" : "=v"(tm) : "v"(__uint_as_float(sw[0])),
          "v"(__uint_as_float(sw[1])));
    }
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
      mc = mn == -INFINITY ? 0.0f : mn * c2;
    }
  };
  // kRel form: sc already holds scale_log2 * score - mc (the QK product
  // started from neg_m), so the lazy test compares with 8 directly. On a
  // rescale a lane moves its reference up by delta = max(tm, 0) (an unset
  // lane to its first tile maximum) and takes delta off this tile's values.
  auto softmax_rescale_rel = [&](f32x16 (&sc)[2], float& l, f32x16 (&O)[DB]) {
    float tm = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) tm = fmaxf(tm, sc[kb][j]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm), __float_as_uint(tm),
                                                       false, false);
      asm("v_max_f32 %0, %1, %2" : "=v"(tm) : "v"(__uint_as_float(sw[0])),
          "v"(__uint_as_float(sw[1])));
    }
    // an unset lane with a finite maximum always rescales
    if (__ballot((tm > 8.0f) | (unset & (tm != -INFINITY))) != 0) {
      // unset: l = 0 and O = 0, so the factor only has to be finite; a lane
      // still without an allowed key (tm = -inf) stays unset with delta 0
      const float delta = unset ? (tm == -INFINITY ? 0.0f : tm) : fmaxf(tm, 0.0f);
      const float corr = unset ? 1.0f : fast_exp2(-delta);
      l *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) O[db] *= corr;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[kb][j] -= delta;
      mc_f += delta;
      unset = unset & (tm == -INFINITY);
#pragma unroll
      for (int j = 0; j < 16; ++j) neg_m[j] = -mc_f;
      asm volatile("" : "+v"(neg_m));
    }
  };
  auto softmax_weights = [&](const f32x16 (&sc)[2], float mc, float& l, E8 (&pb)[4]) {
    float p[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        p[kb][j] = kRel ? fast_exp2(sc[kb][j]) : fast_exp2(fmaf(sc[kb][j], c2, -mc));
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[s][i] = (Elem)p[s >> 1][8 * (s & 1) + i];
    // the row sum adds the rounded values the PV product uses, two per dot2
    // (two chains, the first continuing from l)
    float ls0 = l, ls1 = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 8; i += 4) {
        ls0 = add_pair(E2{pb[s][i], pb[s][i + 1]}, ls0);
        ls1 = add_pair(E2{pb[s][i + 2], pb[s][i + 3]}, ls1);
      }
    l = ls0 + ls1;
  };
  auto softmax_update = [&](f32x16 (&sc)[2], float& m, float& mc, float& l,
                            f32x16 (&O)[DB], E8 (&pb)[4]) {
    if constexpr (kRel)
      softmax_rescale_rel(sc, l, O);
    else
      softmax_rescale(sc, m, mc, l, O);
    softmax_weights(sc, mc, l, pb);
  };
  // V^T fragment of lane (q32, h2) for slice s and d-block db: channel
  // 32 db + q32 of keys 16s + 4 h2 .. + 3 and 16s + 8 + 4 h2 .. + 3. In the
  // direct layout (V rows in LDS) it takes two transposed reads: the 16-lane
  // group (h2, dsub = bit 4 of the lane) reads rows 4 h2 + c / 4 (plus the
  // slice's first key, plus 8 for the second half) at channels
  // 32 db + 16 dsub + 4 (c % 4), c = lane % 16; v_lane is that address for
  // db = 0 and the slice's first key, the segment of block db being an XOR.
  const int c16 = lane & 15, dsub = (lane >> 4) & 1;
  const uint32_t v_lane = (uint32_t)((4 * h2 + (c16 >> 2)) * RB + ((dsub ^ vsw(c16 >> 2)) << 5) +
                                     ((c16 & 3) >> 1) * 16 + (c16 & 1) * 8);
  // The XOR'd lane offsets of the operand reads, computed once. In the
  // gate-blended forward they are kept in registers behind an empty asm the
  // compiler cannot look through: under that mode's register pressure it
  // rebuilt each address with a v_or before every read (48 VALU per tile);
  // the other modes keep them by themselves.
  uint32_t v_off[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    v_off[db] = v_lane ^ (uint32_t)(db << 6);
    if constexpr (kMixed) asm volatile("" : "+v"(v_off[db]));
  }
  auto pv = [&](const uint16_t* vt, const E8 (&pb)[4], f32x16 (&O)[DB]) {
    // all V^T fragments of two 16-key slices are requested before their
    // products (the empty asm keeps the compiler from sinking each read next
    // to its use, which would expose the LDS latency between products)
#pragma unroll
    for (int s2 = 0; s2 < 4; s2 += 2) {
      E8 av[2][DB];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          if constexpr (kDma) {
            const char* p = reinterpret_cast<const char*>(vt) + v_off[db] + 16 * (s2 + h) * RB;
            av[h][db] = __builtin_bit_cast(E8, lds_tr_pair(p, p + 8 * RB));
          } else {
            // keys 16s+4h2..+3 and 16s+8+4h2..+3: one adjacent 16-byte pair
            const int d = 32 * db + q32;
            av[h][db] = as_elem8<kF16>(
                *reinterpret_cast<const u32x4*>(vt + d * kBN + 4 * vt_slot(4 * (s2 + h) + h2, d)));
          }
        }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          O[db] = mma32(av[h][db], pb[s2 + h], O[db]);
    }
  };

  // S^T = K Q^T for the 64 keys of the K tile at ks (two 32-key blocks). All
  // K fragments of a block are requested before its first product (as for V
  // above), and the two blocks' independent accumulation chains are
  // interleaved.
  // K fragment of lane (q32, h2) for k-step ks_: chunk 2 ks_ + h2 of key rows
  // q32 and q32 + 32; in the direct layout at slot (2 ks_ + h2) ^ ksw(q32)
  // (ksw(q32 + 32) = ksw(q32)), an XOR of k_lane by 32 ks_.
  const uint32_t k_lane = (uint32_t)(q32 * RB + ((h2 ^ ksw(q32)) << 4));
  uint32_t k_off[KS];
#pragma unroll
  for (int ks_ = 0; ks_ < KS; ++ks_) {
    k_off[ks_] = k_lane ^ (uint32_t)(ks_ << 5);
    if constexpr (kMixed) asm volatile("" : "+v"(k_off[ks_]));
  }
  auto qk = [&](const uint16_t* ks, f32x16 (&st)[2]) {
    st[0] = kRel ? neg_m : f32x16{};
    st[1] = kRel ? neg_m : f32x16{};
    E8 ak0[KS], ak1[KS];
    if constexpr (kDma) {
      const char* kb = reinterpret_cast<const char*>(ks);
#pragma unroll
      for (int ks_ = 0; ks_ < KS; ++ks_)
        ak0[ks_] = as_elem8<kF16>(*reinterpret_cast<const u32x4*>(kb + k_off[ks_]));
      asm volatile("" ::: "memory");
#pragma unroll
      for (int ks_ = 0; ks_ < KS; ++ks_)
        ak1[ks_] = as_elem8<kF16>(*reinterpret_cast<const u32x4*>(kb + k_off[ks_] + 32 * RB));
      asm volatile("" ::: "memory");
    } else {
      const uint16_t* krow0 = ks + q32 * KPAD + 8 * h2;
      const uint16_t* krow1 = krow0 + 32 * KPAD;
#pragma unroll
      for (int ks_ = 0; ks_ < KS; ++ks_)
        ak0[ks_] = as_elem8<kF16>(*reinterpret_cast<const u32x4*>(krow0 + 16 * ks_));
      asm volatile("" ::: "memory");
#pragma unroll
      for (int ks_ = 0; ks_ < KS; ++ks_)
        ak1[ks_] = as_elem8<kF16>(*reinterpret_cast<const u32x4*>(krow1 + 16 * ks_));
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int ks_ = 0; ks_ < KS; ++ks_) {
      st[0] = mma32(ak0[ks_], qf[ks_], st[0]);
      st[1] = mma32(ak1[ks_], qf[ks_], st[1]);
    }
  };
  // Causal / Lambda mask of tile k's raw scores, in place (unmasked tiles
  // use the product registers as they are: a separate masked copy cost 32
  // moves per tile on the unmasked path). Tiles wholly below the wave's
  // first query need none.
  auto mask_scores = [&](int k, f32x16 (&st)[2]) {
    const int p0 = tile_pos(k);
    const bool lam_phase = kStream || (kTwoPhase && k < nlam);
    const bool diag = p0 + kBN - 1 > i_wfirst;
    if (lam_phase || diag) {
      // Element j of the lane's scores is key base + c_j, with c_j a
      // compile-time offset. One loop per mode (a tile-uniform branch
      // between two loops made the compiler copy the scores at the join on
      // every tile). Bitwise operators: a select per element, no per-lane
      // branches.
      const int base = p0 + 4 * h2;
      if constexpr (kCache || lblk) {
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
      } else if (lam_phase && p0 >= a.S) {
        // token-level Lambda on a tile past the sinks: the window band
        // 0 <= i - j < R, one unsigned compare of dq - c_j against R
        const int dq = i_q - base;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int c = 32 * kb + 8 * (j >> 2) + (j & 3);
            st[kb][j] = (uint32_t)(dq - c) < (uint32_t)a.R ? st[kb][j] : -INFINITY;
          }
      } else {
        // token-level Lambda; outside the Lambda phase every key passes the
        // sink test, leaving the causal one
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
  };
  // Masked scores, softmax update and PV product of tile k from its raw
  // scores st and V tile vt; tiles wholly above the wave's last query are
  // skipped.
  auto consume = [&](int k, f32x16 (&st)[2], const uint16_t* vt) {
    if (tile_pos(k) <= i_wlast) {
      mask_scores(k, st);
      E8 pb[4];
      softmax_update(st, m_f, mc_f, l_f, o_f, pb);
      pv(vt, pb, o_f);
    }
  };
  // End of the Lambda phase of the two-phase modes: keep (1 - alpha) * O / l
  // (forward) or dout . O / l (gate gradient), restart the state.
  auto end_lambda_phase = [&]() {
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
    mc_f = 0.0f;
    l_f = 0.0f;
    if constexpr (kRel) {
      unset = true;
      neg_m = f32x16{};
      asm volatile("" : "+v"(neg_m));
    }
  };

  // ---- main loop ----------------------------------------------------------------
  {
    if constexpr (kDma) {
      dma_rows(tile_pos(0), Ks0, krs, k_c16, k_lo);
      dma_rows(tile_pos(0), Vs0, vrs, v_c16, v_lo);
    } else {
      load_tile(tile_pos(0));
      store_tile(Ks0, Vs0);
    }
    __syncthreads();
    // Every load issued so far (the query fragments, tile 0) has landed: say
    // so explicitly. Without it the wait-count insertion merges the path on
    // which no tile store waited into the loop header and keeps the query
    // loads "pending", so each iteration's QK products would wait for the
    // next tile's prefetch (vmcnt counts in order), exposing its whole
    // latency.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    // One tile from stage S = k & 1 (a compile-time constant): the next
    // tile's loads go to the other stage, which was last read before the
    // previous barrier. Direct loads complete before the barrier that ends
    // the step (the barrier waits for the wave's outstanding loads).
    auto step = [&](int k, auto stage) {
      constexpr int S = decltype(stage)::value;
      uint16_t* ks = S ? Ks1 : Ks0;
      uint16_t* vs = S ? Vs1 : Vs0;
      uint16_t* ks_next = S ? Ks0 : Ks1;
      uint16_t* vs_next = S ? Vs0 : Vs1;
      const bool more = k + 1 < ntiles;
      if (more) {
        if constexpr (kDma) {
          dma_rows(tile_pos(k + 1), ks_next, krs, k_c16, k_lo);
          dma_rows(tile_pos(k + 1), vs_next, vrs, v_c16, v_lo);
        } else {
          load_tile(tile_pos(k + 1));
        }
      }
      if (kTwoPhase && k == nlam) end_lambda_phase();
      f32x16 st[2];
      qk(ks, st);
      consume(k, st, vs);
      if constexpr (!kDma) {
        if (more) store_tile(ks_next, vs_next);
      }
      __syncthreads();
    };
    for (int k = 0; k < ntiles; k += 2) {
      step(k, std::integral_constant<int, 0>());
      if (k + 1 < ntiles) step(k + 1, std::integral_constant<int, 1>());
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
  // The wave's 32 output rows (its tokens of one head) go through LDS, so the
  // stores are whole rows, 64 / (D/8) rows per instruction, instead of 16
  // bytes in each of 32 rows (Hq*D*2 bytes apart) per instruction. The tile
  // stages are free after the loop's last barrier; each wave uses 32*D
  // elements of one of them (16-byte chunks XOR-swizzled by row). Rows of
  // tokens past the chunk are staged but not stored.
  const float lf = l_f + __shfl_xor(l_f, 32, 64);
  const float wf = alpha / lf;  // alpha = 1 outside the mixed forward
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  static_assert(2 * 32 * D <= kBN * KROW && 2 * 32 * D <= D * kBN, "two waves per stage");
  uint16_t* stg = (wave < 2 ? Ks0 : wave < 4 ? Ks1 : wave < 6 ? Vs0 : Vs1) + (wave & 1) * 32 * D;
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
      const int ch = (4 * db + jb) ^ (q32 & (CPR - 1));  // channels 32 db + 8 jb ..
      *reinterpret_cast<uint2*>(stg + q32 * D + 8 * ch + 4 * h2) = w;
    }
  __syncthreads();
  constexpr int RPS = 64 / CPR;  // rows per store instruction
  const int lr = lane / CPR, lc = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPS; ++i) {
    const int row = i * RPS + lr, tok = w_tok0 + row;
    const u32x4 val =
        *reinterpret_cast<const u32x4*>(stg + row * D + 8 * (lc ^ (row & (CPR - 1))));
    if (tok < a.T) st16(a.out + (((int64_t)b * a.T + tok) * a.Hq + head) * D + 8 * lc, val);
  }
}

template <int D, int HB, int MODE>
__global__ __launch_bounds__(64 * attn_waves<MODE>(), 1) void attn_kernel(AttnArgs a) {
  attn_body<D, HB, MODE, true>(a);
}
template <int D, int HB, int MODE>
__global__ __launch_bounds__(64 * attn_waves<MODE>(), 1) void attn_kernel_exact(AttnArgs a) {
  attn_body<D, HB, MODE, false>(a);
}

// DUO_EXACT_SCALE=1 in the environment (read at every launch) selects the
// fp32-scale form of the modes that otherwise pre-scale q.
static bool exact_scale_requested() {
  const char* e = getenv("DUO_EXACT_SCALE");
  return e != nullptr && e[0] == '1';
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
  x.tiles_in_y = !mode_streaming(MODE) && x.n_qtiles <= 65535;
  dim3 grid(x.tiles_in_y ? hgs : (unsigned)x.n_qtiles, x.tiles_in_y ? (unsigned)x.n_qtiles : hgs,
            (unsigned)B);
  if constexpr (mode_prescale(MODE)) {
    if (exact_scale_requested()) {
      attn_kernel_exact<D, HB, MODE><<<grid, 64 * NW, 0, s>>>(x);
      return hipGetLastError();
    }
  }
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
  const int D = L->d.head_dim;
  if (L->d.retrieval_dtype == DUO_INT4_G32) {
    a.kcodes = reinterpret_cast<const uint8_t*>(L->rbuf + L->lay.k_offset);
    a.vcodes = reinterpret_cast<const uint8_t*>(L->rbuf + L->lay.v_offset);
    a.ksz = reinterpret_cast<const uint32_t*>(L->rbuf + L->lay.k_sz_offset);
    a.vsz = reinterpret_cast<const uint32_t*>(L->rbuf + L->lay.v_sz_offset);
    a.cap32 = cap32_of(L->d.retrieval_capacity);
    return launch_mode<MODE_RETRIEVAL_I4>(a, D, L->Hr, L->d.batch, s);
  }
  return L->d.retrieval_dtype == DUO_FP16
             ? launch_mode<MODE_RETRIEVAL_F16>(a, D, L->Hr, L->d.batch, s)
             : launch_mode<MODE_RETRIEVAL>(a, D, L->Hr, L->d.batch, s);
}

hipError_t launch_prefill_streaming(const duo_layer* L, const void* q, const void* k,
                                    const void* v, int T, void* out, hipStream_t s) {
  AttnArgs a = base_args(L, q, T, out);
  a.k_in = static_cast<const uint16_t*>(k);
  a.v_in = static_cast<const uint16_t*>(v);
  a.kv_base = L->Hr;
  return L->d.kv_dtype == DUO_FP16
             ? launch_mode<MODE_STREAMING_F16>(a, L->d.head_dim, L->Hs, L->d.batch, s)
             : launch_mode<MODE_STREAMING>(a, L->d.head_dim, L->Hs, L->d.batch, s);
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

// Partials of the allocation-free gate gradient: one fp32 sum per flash block,
// in a file-scope device array instead of a caller workspace. Every device the
// library runs on holds its own copy until the process ends; every call on a
// device shares it, so calls that overlap on one device race.
static __device__ __align__(256) float scratch[kGradScratchPartials];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

// Device address of the current device's copy of `scratch`, looked up once per
// device (with that device current). In host code the array's name is only a
// stand-in: kernels must be given this address.
hipError_t grad_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
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
