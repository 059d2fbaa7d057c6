// Decode attention of a grouped-query KV head on the matrix cores.
//
// With G query heads per KV head every cached row enters G dot products and G
// weighted sums; on the VALU that is 2 G multiply-adds per channel and row,
// which makes the decode loop of G >= 4 layers arithmetic-bound well below the
// HBM rate. Here the G heads are the columns of one v_mfma_f32_32x32x16 tile
// (bf16, or fp16 for an fp16 cache), the rest of the 32 columns zero:
//   S^T = K Q^T   A = 32 key rows x 16 channels, B = Q^T (column = head);
//   O^T += V^T P^T A = 32 channels x 16 keys (transposed LDS reads),
//                  B = the packed softmax weights P^T.
// The operand layouts are the flash kernel's (k_attn.hip): K rows in LDS with
// 16-byte chunks XOR-swizzled by row, V rows with 32-byte segments swizzled by
// row, a lane holding one head's scores for 16 of a tile's keys, and the score
// accumulator reused as the PV operand after a key permutation inside each
// 16-key slice. Each wave streams its own 32-row tiles (rows r0 + 32 w +
// 32 NW k) from global memory straight into a private pair of LDS stages
// (16-byte buffer loads with the LDS bit; the next tile's loads are in flight
// while the current one is computed), so the waves need no barrier. The
// softmax keeps a lazy reference maximum as the flash kernel does; the wave's
// (m, l, O) end in the block's reduction buffer in the log2 domain.
//
// What is computed: the full softmax attention of the retrieval heads over
// their cache (xllm-io review "DuoAttention: Efficient Long-Context LLM
// Inference with Retrieval and Streaming Heads", section 三, 核心公式), for a
// split-K range of rows; the split states are merged as in the VALU path.
#pragma once
#include "decode_common.hpp"
#include "mfma_common.hpp"

namespace duo {

// Rows per wave tile of the matrix-core decode.
constexpr int kMmaRows = 32;

// Attend the G query heads whose rows start at q_heads ([G][D] bf16) over
// cache rows [r0, r1) of kc/vc (head bases; every row offset below 2^31 bytes),
// plus the new token (knew, vnew) in wave 0 when with_new. k0/k1/v0/v1 are
// this wave's two K and two V stages of kMmaRows * D elements each; they must
// point into four distinct __shared__ arrays. c2 = softmax scale * log2(e).
// On return the wave's state is in red.m/l/acc[wave] (callers then run
// block_merge_lds).
template <int D, int G, typename Tag, int NW>
__device__ __forceinline__ void attend_cache_mma(BlockRed<D, G, NW>& red,
                                                 const uint16_t* q_heads, float c2,
                                                 const uint16_t* kc, const uint16_t* vc,
                                                 int r0, int r1,
                                                 const uint16_t* knew, const uint16_t* vnew,
                                                 bool with_new, uint16_t* k0, uint16_t* k1,
                                                 uint16_t* v0, uint16_t* v1) {
  constexpr bool F16 = !Tag::is_bf16;
  using E8 = elem8<F16>;
  using E2 = std::conditional_t<F16, f16x2, bf16x2>;
  using Elem = std::conditional_t<F16, _Float16, __bf16>;
  static_assert(D == 64 || D == 128, "128- or 256-byte rows");
  static_assert(G <= 32, "the heads of a KV head are the columns of one tile");
  constexpr int KS = D / 16;           // k-steps of the QK product
  constexpr int DB = D / 32;           // 32-channel blocks of the PV product
  constexpr int RB = 2 * D;            // bytes per row (LDS rows unpadded)
  constexpr int SPR = RB / 16;         // 16-byte slots per row
  constexpr int RPI = 1024 / RB;       // rows per 1 KB load
  constexpr int NL = kMmaRows / RPI;   // loads per tile and tensor
  constexpr int JK = RB == 256 ? 4 : 2;  // distinct K lane offsets over the loads
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int q32 = lane & 31, h2 = lane >> 5;
  // chunk swizzles (the flash kernel's): K chunk c of row r at slot c ^ ksw(r),
  // V 32-byte segment g of row r at segment g ^ vsw(r)
  auto ksw = [](int r) { return RB == 256 ? (r & 15) : ((r >> 1) & 7); };
  auto vsw = [](int r) { return RB == 256 ? 2 * (r & 3) : (r & 3); };

  // ---- query fragments: lane (q32, h2) holds channels 16 ks + 8 h2 .. + 7 of
  // head q32 (zero for columns past G) ----------------------------------------
  E8 qf[KS];
  {
    const bool act = q32 < G;
    const uint16_t* qp = q_heads + (act ? q32 : 0) * D + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = ld16(qp + 16 * ks);
      if (!act) w = u32x4{0u, 0u, 0u, 0u};
      if constexpr (F16) {
        // bf16 -> fp32 (exact) -> fp16
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t wi = word_of(w, i >> 1);
          qf[ks][i] = (_Float16)__uint_as_float((i & 1) ? (wi & 0xffff0000u) : (wi << 16));
        }
      } else {
        qf[ks] = as_bf16x8(w);
      }
    }
  }

  // ---- direct loads of one 32-row tile into a stage ------------------------------
  // Load j covers tile rows j*RPI .. + RPI - 1; lane i writes LDS slot i of the
  // load's 1 KB (row j*RPI + i/SPR, slot i%SPR) and so fetches the source chunk
  // that belongs there (lane offsets precomputed per load). The tile's rows up
  // to r1 are one buffer resource built in scalar registers: lanes past r1 are
  // out of its range and write zeros to LDS (keys masked, values finite), so no
  // address arithmetic runs per tile and no load leaves the head's rows.
  const int rl = lane / SPR, pos = lane % SPR;
  uint32_t kvo[NL], vvo[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    kvo[j] = (uint32_t)(j * 1024 + rl * RB + 16 * (pos ^ ksw(j * RPI + rl)));
    vvo[j] = (uint32_t)(j * 1024 + rl * RB + 16 * (2 * ((pos >> 1) ^ vsw(rl)) + (pos & 1)));
  }
  auto dma = [&](int t, uint16_t* ks, uint16_t* vs) {
    const int nrow = r1 - t < 0 ? 0 : r1 - t < kMmaRows ? r1 - t : kMmaRows;  // wave-uniform
    const uint32_t nbytes = (uint32_t)(nrow * RB);
    const __amdgpu_buffer_rsrc_t krs = wave_rsrc(kc + (int64_t)t * D, nbytes);
    const __amdgpu_buffer_rsrc_t vrs = wave_rsrc(vc + (int64_t)t * D, nbytes);
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, lds_ptr(ks + j * 512), 16, (int)kvo[j], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, lds_ptr(vs + j * 512), 16, (int)vvo[j], 0, 0, 0);
    }
  };

  // ---- operand reads (flash-kernel addressing for a 32-row tile) ----------------
  // K fragment of k-step ks: chunk 2 ks + h2 of key row q32.
  const uint32_t k_lane = (uint32_t)(q32 * RB + ((h2 ^ ksw(q32)) << 4));
  // V^T fragment of slice s (keys 16 s ..) and d-block db: two transposed reads
  // of rows 4 h2 + c16 / 4 (+ 8) at channels 32 db + 16 dsub + 4 (c16 % 4).
  const int c16 = lane & 15, dsub = (lane >> 4) & 1;
  const uint32_t v_lane = (uint32_t)((4 * h2 + (c16 >> 2)) * RB + ((dsub ^ vsw(c16 >> 2)) << 5) +
                                     ((c16 & 3) >> 1) * 16 + (c16 & 1) * 8);

  // ---- state ------------------------------------------------------------------------
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = -INFINITY, mc = 0.0f, l = 0.0f;  // m in raw score units, mc = m * c2
  const float lazy = 8.0f / c2;              // raw-score growth that forces a rescale

  auto compute = [&](int t, const uint16_t* ks, const uint16_t* vs) {
    f32x16 st = f32x16{};
    {
      const char* kb = reinterpret_cast<const char*>(ks);
      E8 ak[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        ak[s] = as_elem8<F16>(*reinterpret_cast<const u32x4*>(kb + (k_lane ^ (uint32_t)(s << 5))));
#pragma unroll
      for (int s = 0; s < KS; ++s) st = mma32(ak[s], qf[s], st);
    }
    // element j of the lane's scores is key t + 4 h2 + 8 (j / 4) + j % 4
    if (t + kMmaRows > r1) {  // the tile reaching past r1 (wave-uniform)
      const int lim = r1 - t - 4 * h2;
#pragma unroll
      for (int j = 0; j < 16; ++j) st[j] = 8 * (j >> 2) + (j & 3) < lim ? st[j] : -INFINITY;
    }
    float tm = st[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) tm = fmaxf(tm, st[j]);
    // lanes l and l + 32 hold the two halves of a head's keys: one
    // v_permlane32_swap gives every lane its partner's maximum
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tm), __float_as_uint(tm),
                                                       false, false);
      tm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    if (__ballot(tm > m + lazy) != 0) {
      // every tile holds a key below r1, so mn is finite; m = -inf gives 0
      const float mn = fmaxf(m, tm);
      const float corr = fast_exp2((m - mn) * c2);
      l *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= corr;
      m = mn;
      mc = mn * c2;
    }
    E8 pb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[s][i] = (Elem)fast_exp2(fmaf(st[8 * s + i], c2, -mc));
    // row sum of the rounded weights the PV product uses
    float ls0 = l, ls1 = 0.0f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 8; i += 4) {
        ls0 = add_pair(E2{pb[s][i], pb[s][i + 1]}, ls0);
        ls1 = add_pair(E2{pb[s][i + 2], pb[s][i + 3]}, ls1);
      }
    l = ls0 + ls1;
    const char* vb = reinterpret_cast<const char*>(vs);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      E8 av[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* p = vb + (v_lane ^ (uint32_t)(db << 6)) + 16 * s * RB;
        av[db] = __builtin_bit_cast(E8, lds_tr_pair(p, p + 8 * RB));
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = mma32(av[db], pb[s], o[db]);
    }
  };

  // ---- the wave's tiles: two stages, the next tile's loads in flight ----------------
  // The prefetch is issued even past the range (its resource is empty, so the
  // stage fills with zeros and is never computed): every step issues the same
  // loads, and the compiler's wait before a stage's reads covers that stage only.
  constexpr int stride = kMmaRows * NW;
  int t = r0 + kMmaRows * wave;
  if (t < r1) {
    dma(t, k0, v0);
    for (;;) {
      const int t1 = t + stride;
      dma(t1, k1, v1);
      compute(t, k0, v0);
      if (t1 >= r1) break;
      t = t1 + stride;
      dma(t, k0, v0);
      compute(t1, k1, v1);
      if (t >= r1) break;
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // no load into LDS outlives the loop
  }

  // ---- the new token (read from its input), one more key in wave 0 -------------------
  if (with_new && wave == 0) {
    float d = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float kf[8];
      unpack8<Tag>(ld16(knew + 16 * s + 8 * h2), kf);
#pragma unroll
      for (int i = 0; i < 8; ++i) d = fmaf((float)qf[s][i], kf[i], d);
    }
    d += __shfl_xor(d, 32, 64);
    const float mn = fmaxf(m, d);
    const float corr = fast_exp2((m - mn) * c2);  // m = -inf: 0 (l and o are 0)
    const float p = fast_exp2((d - mn) * c2);
    l = l * corr + (h2 == 0 ? p : 0.0f);          // l is split over the lane pair
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const uint2 w = *reinterpret_cast<const uint2*>(vnew + 32 * db + 8 * jb + 4 * h2);
        float vf[4];
        if constexpr (F16) {
          vf[0] = f16lo(w.x); vf[1] = f16hi(w.x); vf[2] = f16lo(w.y); vf[3] = f16hi(w.y);
        } else {
          vf[0] = bf16lo(w.x); vf[1] = bf16hi(w.x); vf[2] = bf16lo(w.y); vf[3] = bf16hi(w.y);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) o[db][4 * jb + r] = fmaf(p, vf[r], o[db][4 * jb + r] * corr);
      }
    m = mn;
  }

  // ---- the wave's state, log2 domain, into the block's reduction buffer --------------
  // element (db, 4 jb + r) of o is channel 32 db + 8 jb + 4 h2 + r of head q32
  const float lt = l + __shfl_xor(l, 32, 64);
  if (q32 < G) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        float4 v4 = make_float4(o[db][4 * jb], o[db][4 * jb + 1], o[db][4 * jb + 2],
                                o[db][4 * jb + 3]);
        *reinterpret_cast<float4*>(&red.acc[wave][q32][32 * db + 8 * jb + 4 * h2]) = v4;
      }
    if (h2 == 0) {
      red.m[wave][q32] = m == -INFINITY ? -INFINITY : m * c2;
      red.l[wave][q32] = lt;
    }
  }
}

}  // namespace duo
