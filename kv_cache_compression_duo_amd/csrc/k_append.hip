// Cache-append kernels: retrieval rows (verbatim or 4-bit group encoded), ring
// slots of the streaming heads, and a zero-fill used for the workspace.
//
// The two caches per layer and the split of new K/V along the head axis follow
// the xllm-io review "DuoAttention: Efficient Long-Context LLM Inference with
// Retrieval and Streaming Heads", section 三 推理流程. The 4-bit encoding is
// this library's reading of the 4-bit KV cache the same page names in section
// 五 量化组合: per token, head and 32-channel group, fp16 scale
// s = (max - min) / 15 and fp16 zero-point z = min, codes
// rint((x - z) / s) clamped to [0, 15] (0 when s == 0), all in fp32 with IEEE
// division so that the codes are reproducible bit for bit.
#include "device_common.hpp"
#include "duo_internal.hpp"
#include "int4_codec.hpp"

namespace duo {

// ---- verbatim retrieval rows -------------------------------------------------
// One thread per 16-byte chunk: k/v [B][T][Hkv][D] -> cache [B][Hr][cap][D].
// A block covers 256 / chunks consecutive tokens of one (sequence, head);
// grid (token groups, Hr, B), chunks a power of two: no index division.
__global__ void append_rows_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                   u32x4* __restrict__ kc, u32x4* __restrict__ vc, int T,
                                   int Hkv, int Hr, int lchunks, int64_t cap, int64_t n) {
  const int chunks = 1 << lchunks;
  const int c = (int)threadIdx.x & (chunks - 1);
  const int t = (int)blockIdx.x * ((int)blockDim.x >> lchunks) + ((int)threadIdx.x >> lchunks);
  if (t >= T) return;
  const int h = (int)blockIdx.y, b = (int)blockIdx.z;
  const int64_t src = (((int64_t)b * T + t) * Hkv + h) * chunks + c;
  const int64_t dst = (((int64_t)b * Hr + h) * cap + n + t) * chunks + c;
  kc[dst] = k[src];
  vc[dst] = v[src];
}

// 4-bit cache append. Key codes are token-major ([cap32][D/2] bytes, byte b of
// a row = channel 2b | channel 2b+1 << 4). Value codes are stored in 32-token
// blocks of 16*D bytes laid out in the operand order of the decode kernel's PV
// product: for channel ch and m in [0, 16), the byte at
//   16 * (4 * (16 * (ch / 64) + ch % 16) + m / 4) + 4 * ((ch % 64) / 16) + m % 4
// holds token m of the block in its low nibble and token m + 16 in its high
// nibble. Scale and zero-point words (fp16 s | fp16 z << 16) are blocked the
// same way: [cap32/32][D/32][32], word t % 32 of group g of block t / 32.
// A thread owns one byte position m of a block (tokens m and m + 16) and 8
// channels, so no two threads write the same byte; a byte whose other token
// lies outside the appended range is read, modified and written by its one
// owner.
// Thread order: channel chunk fastest, so the 4 lanes of a quad hold one
// 32-channel group of one token (the min/max reduction uses quad DPP).
template <typename Tag>
__global__ void append_int4_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                   uint32_t* __restrict__ kcodes, uint8_t* __restrict__ vcodes,
                                   uint32_t* __restrict__ ksz, uint32_t* __restrict__ vsz, int B,
                                   int T, int Hkv, int Hr, int chunks, int64_t cap32, int64_t n,
                                   int64_t blk0, int nblk) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)B * Hr * nblk * 16 * chunks;
  if (i >= total) return;  // whole quads: total and blockDim are multiples of 4
  const int c = (int)(i % chunks);
  int64_t r = i / chunks;
  const int m = (int)(r % 16);
  r /= 16;
  const int64_t blk = blk0 + r % nblk;
  r /= nblk;
  const int h = (int)(r % Hr);
  const int b = (int)(r / Hr);
  const int64_t hb = (int64_t)b * Hr + h;
  const int groups = chunks / 4;
  const int D = chunks * 8;
  uint32_t vq[2] = {0u, 0u};
  bool in[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t p = blk * 32 + m + 16 * e;
    in[e] = p >= n && p < n + T;  // uniform over the quad (same token)
    if (in[e]) {
      const int64_t src = (((int64_t)b * T + (p - n)) * Hkv + h) * chunks + c;
      uint32_t kq, ks, vs;
      encode_group_part<Tag>(k[src], &kq, &ks);
      encode_group_part<Tag>(v[src], &vq[e], &vs);
      const int64_t row = hb * cap32 + p;
      kcodes[row * chunks + c] = kq;
      if ((c & 3) == 0) {
        const int64_t w = ((hb * (cap32 / 32) + p / 32) * groups + c / 4) * 32 + p % 32;
        ksz[w] = ks;
        vsz[w] = vs;
      }
    }
  }
  if (!in[0] && !in[1]) return;  // this byte pair lies outside the appended range
  // value codes of channels ch = 8c + j, j < 8: the bytes for consecutive j
  // are 64 apart (ch % 16 steps by one)
  uint8_t* vb = vcodes + (hb * (cap32 / 32) + blk) * 16 * D +
                16 * (4 * (16 * (c / 8) + 8 * (c % 2)) + m / 4) + 4 * ((c % 8) / 2) + m % 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint8_t* dst = vb + 64 * j;
    const uint32_t lo = (vq[0] >> (4 * j)) & 0xFu, hi = (vq[1] >> (4 * j)) & 0xFu;
    uint32_t byte;
    if (in[0] && in[1]) {
      byte = lo | (hi << 4);
    } else {
      const uint32_t old = *dst;
      byte = in[0] ? (old & 0xF0u) | lo : (old & 0x0Fu) | (hi << 4);
    }
    *dst = (uint8_t)byte;
  }
}

// ---- ring slots --------------------------------------------------------------
// Writes the positions of [n, n+T) that survive the chunk: those < S and the
// last R positions >= S. They land in distinct slots, so threads never collide.
__global__ void append_ring_kernel(const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                   u32x4* __restrict__ kr, u32x4* __restrict__ vr, int B, int T,
                                   int Hkv, int Hr, int Hs, int chunks, int S, int R, int64_t n,
                                   int cnt_sink, int64_t lo_recent, int cnt_recent) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int cnt = cnt_sink + cnt_recent;
  int64_t total = (int64_t)B * cnt * Hs * chunks;
  if (i >= total) return;
  int c = (int)(i % chunks);
  int64_t r = i / chunks;
  int hs = (int)(r % Hs);
  r /= Hs;
  int e = (int)(r % cnt);
  int b = (int)(r / cnt);
  int64_t p = e < cnt_sink ? n + e : lo_recent + (e - cnt_sink);
  int slot = p < S ? (int)p : S + (int)((p - S) % R);
  int t = (int)(p - n);
  int64_t src = (((int64_t)b * T + t) * Hkv + Hr + hs) * chunks + c;
  int64_t dst = (((int64_t)b * Hs + hs) * (S + R) + slot) * chunks + c;
  kr[dst] = k[src];
  vr[dst] = v[src];
}

__global__ void zero_kernel(u32x4* p, int64_t n16) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = u32x4{0u, 0u, 0u, 0u};
}

static inline unsigned blocks_for(int64_t n, int t) { return (unsigned)((n + t - 1) / t); }

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  zero_kernel<<<blocks_for(n16, 256), 256, 0, s>>>(static_cast<u32x4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_append_cache(const duo_layer* L, const void* k, const void* v, int T,
                               hipStream_t s) {
  const duo_layer_desc& d = L->d;
  int chunks = d.head_dim / 8;
  int64_t total = (int64_t)d.batch * T * L->Hr * chunks;
  if (total == 0) return hipSuccess;
  if (d.retrieval_dtype == DUO_INT4_G32) {
    const int64_t cap32 = cap32_of(d.retrieval_capacity);
    const int64_t blk0 = L->n / 32, blk1 = (L->n + T - 1) / 32;
    const int nblk = (int)(blk1 - blk0 + 1);
    const int64_t tot = (int64_t)d.batch * L->Hr * nblk * 16 * chunks;
    auto* kq = reinterpret_cast<uint32_t*>(L->rbuf + L->lay.k_offset);
    auto* vq = reinterpret_cast<uint8_t*>(L->rbuf + L->lay.v_offset);
    auto* ks = reinterpret_cast<uint32_t*>(L->rbuf + L->lay.k_sz_offset);
    auto* vs = reinterpret_cast<uint32_t*>(L->rbuf + L->lay.v_sz_offset);
    const unsigned g4 = blocks_for(tot, 256);
    if (d.kv_dtype == DUO_FP16)
      append_int4_kernel<Fp16Tag><<<g4, 256, 0, s>>>(
          static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), kq, vq, ks, vs, d.batch, T,
          d.n_kv_heads, L->Hr, chunks, cap32, L->n, blk0, nblk);
    else
      append_int4_kernel<Bf16Tag><<<g4, 256, 0, s>>>(
          static_cast<const u32x4*>(k), static_cast<const u32x4*>(v), kq, vq, ks, vs, d.batch, T,
          d.n_kv_heads, L->Hr, chunks, cap32, L->n, blk0, nblk);
  } else {
    // grid dimensions y and z hold at most 65535 blocks
    if (L->Hr > 65535 || d.batch > 65535) return hipErrorInvalidValue;
    const int lchunks = chunks == 16 ? 4 : 3;  // head_dim 128 or 64
    const int per_block = 256 >> lchunks;
    const dim3 g3((unsigned)((T + per_block - 1) / per_block), (unsigned)L->Hr, (unsigned)d.batch);
    append_rows_kernel<<<g3, 256, 0, s>>>(
        static_cast<const u32x4*>(k), static_cast<const u32x4*>(v),
        reinterpret_cast<u32x4*>(L->rbuf + L->lay.k_offset),
        reinterpret_cast<u32x4*>(L->rbuf + L->lay.v_offset), T, d.n_kv_heads, L->Hr, lchunks,
        d.retrieval_capacity, L->n);
  }
  return hipGetLastError();
}

hipError_t launch_append_ring(const duo_layer* L, const void* k, const void* v, int T,
                              hipStream_t s) {
  const duo_layer_desc& d = L->d;
  const int64_t n = L->n, S = d.sink, R = d.recent;
  // sinks among the chunk: positions [n, min(S, n+T))
  int64_t sink_hi = n + T < S ? n + T : S;
  int cnt_sink = sink_hi > n ? (int)(sink_hi - n) : 0;
  // last R positions at or after S: [max(S, n, n+T-R), n+T)
  int64_t lo = n + T - R;
  if (lo < S) lo = S;
  if (lo < n) lo = n;
  int cnt_recent = n + T > lo ? (int)(n + T - lo) : 0;
  int chunks = d.head_dim / 8;
  int64_t total = (int64_t)d.batch * (cnt_sink + cnt_recent) * L->Hs * chunks;
  if (total == 0) return hipSuccess;
  append_ring_kernel<<<blocks_for(total, 256), 256, 0, s>>>(
      static_cast<const u32x4*>(k), static_cast<const u32x4*>(v),
      reinterpret_cast<u32x4*>(L->sbuf + L->lay.ring_k_offset),
      reinterpret_cast<u32x4*>(L->sbuf + L->lay.ring_v_offset), d.batch, T, d.n_kv_heads, L->Hr,
      L->Hs, chunks, d.sink, d.recent, n, cnt_sink, lo, cnt_recent);
  return hipGetLastError();
}

}  // namespace duo
