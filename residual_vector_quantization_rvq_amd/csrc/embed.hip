// embed.hip -- one embedding row per token of a mixed text / visual sequence.
//
// "LongCat-2.5 发布：面向智能体任务的原生多模态大模型", section "Visual
// Primitive Modeling": visual signals become multi-level discrete tokens
// that the backbone takes in the same token format as text, and (paragraph
// "Native Visual Representation") the visual codebook embeddings are learned
// jointly with the backbone.  A visual token's embedding is the sum of its
// rows in the L per-level embedding tables -- the decode's gather-sum, over
// tables of the model width -- and a text token's is one row of the text
// embedding table.
//
// HBM/MALL-bound gather.  One wave per token; whether the token is visual is
// a wave-uniform load.  Every lane takes pieces of 8 features: a visual
// token issues the gathers of up to 8 levels before adding them in level
// order in fp32 (bit for bit the decode's sum), a text token copies its row.
// Out-of-range IDs add nothing (a text token's row is then zero) and are
// counted.
#include "common.h"

namespace rvq {

namespace {

typedef float emb_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t emb_u32x4 __attribute__((ext_vector_type(4)));

// eight features of a table row as fp32 (bf16 widens exactly)
__device__ __forceinline__ void load8(const float *row, int c, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4 *>(row)[2 * c];
  const float4 b = reinterpret_cast<const float4 *>(row)[2 * c + 1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t *row, int c, float (&v)[8]) {
  const uint4 q = reinterpret_cast<const uint4 *>(row)[c];
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}
__device__ __forceinline__ float load1(const float *row, int i) { return row[i]; }
__device__ __forceinline__ float load1(const uint16_t *row, int i) {
  return bf16_bits_to_f32(row[i]);
}

// output pieces: fp32 as is, bf16 rounded to nearest even; non-temporal, so
// the output stream does not evict the tables from the caches
__device__ __forceinline__ void store8(float *o, int c, const float (&v)[8]) {
  const emb_f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<emb_f32x4 *>(o) + 2 * c);
  __builtin_nontemporal_store(b, reinterpret_cast<emb_f32x4 *>(o) + 2 * c + 1);
}
__device__ __forceinline__ void store8(uint16_t *o, int c, const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = (uint32_t)f32_to_bf16_bits(v[2 * e]) | ((uint32_t)f32_to_bf16_bits(v[2 * e + 1]) << 16);
  const emb_u32x4 q = {w[0], w[1], w[2], w[3]};
  __builtin_nontemporal_store(q, reinterpret_cast<emb_u32x4 *>(o) + c);
}
__device__ __forceinline__ void store1(float *o, int i, float v) { o[i] = v; }
__device__ __forceinline__ void store1(uint16_t *o, int i, float v) { o[i] = f32_to_bf16_bits(v); }

}  // namespace

// VEC: D is a multiple of 8, so every 8-feature piece of a row is 16-byte
// aligned in both table types and both output types.
template <typename TabT, typename OutT, bool VEC>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t *__restrict__ ids,
                                                    const uint8_t *__restrict__ is_visual,
                                                    int64_t T, int L, const TabT *__restrict__ text,
                                                    int64_t V, const TabT *__restrict__ vis, int K,
                                                    int D, OutT *__restrict__ out,
                                                    uint32_t *__restrict__ bad) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;  // wave-uniform
  if (t >= T) return;
  const int32_t *tid = ids + t * L;
  const bool visual = is_visual == nullptr || is_visual[t] != 0;
  const int id0 = tid[0];
  const bool text_ok = id0 >= 0 && (int64_t)id0 < V;
  if (bad) {  // L <= 64, checked on the host
    if (visual) {
      const int my = lane < L ? tid[lane] : 0;
      const unsigned long long m = __ballot(my < 0 || my >= K);
      if (lane == 0 && m) atomicAdd(bad, (uint32_t)__popcll(m));
    } else if (lane == 0 && !text_ok) {
      atomicAdd(bad, 1u);
    }
  }
  OutT *o = out + t * D;
  if (VEC) {
    const int pieces = D >> 3;
    if (visual) {
      for (int c = lane; c < pieces; c += 64) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int l0 = 0; l0 < L; l0 += 8) {
          float v[8][8];
          bool ok[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int l = l0 + u;
            const int id = l < L ? tid[l] : -1;
            ok[u] = id >= 0 && id < K;
            if (ok[u]) {
              load8(vis + ((int64_t)l * K + id) * D, c, v[u]);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (ok[u]) {  // level order; skipped levels add nothing
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[e] += v[u][e];
            }
        }
        store8(o, c, acc);
      }
    } else {
      const TabT *row = text + (text_ok ? (int64_t)id0 * D : 0);
      for (int c = lane; c < pieces; c += 64) {
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (text_ok) load8(row, c, v);
        store8(o, c, v);
      }
    }
  } else {
    for (int i = lane; i < D; i += 64) {
      float acc = 0.f;
      if (visual) {
        for (int l = 0; l < L; ++l) {
          const int id = tid[l];
          if (id >= 0 && id < K) acc += load1(vis + ((int64_t)l * K + id) * D, i);
        }
      } else if (text_ok) {
        acc = load1(text + (int64_t)id0 * D, i);
      }
      store1(o, i, acc);
    }
  }
}

hipError_t launch_embed(const int32_t *ids, const uint8_t *is_visual, int64_t T, int L,
                        const void *text, int64_t V, const void *vis, int K, int D, bool tab_bf16,
                        void *out, bool out_bf16, uint32_t *bad, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(T, 4)), block(256);
  const bool vec = (D & 7) == 0;
#define RVQ_EMBED(TT, OT, VV)                                                                    \
  embed_kernel<TT, OT, VV><<<grid, block, 0, s>>>(ids, is_visual, T, L, (const TT *)text, V,     \
                                                  (const TT *)vis, K, D, (OT *)out, bad)
  if (tab_bf16) {
    if (out_bf16) {
      if (vec) RVQ_EMBED(uint16_t, uint16_t, true); else RVQ_EMBED(uint16_t, uint16_t, false);
    } else {
      if (vec) RVQ_EMBED(uint16_t, float, true); else RVQ_EMBED(uint16_t, float, false);
    }
  } else {
    if (out_bf16) {
      if (vec) RVQ_EMBED(float, uint16_t, true); else RVQ_EMBED(float, uint16_t, false);
    } else {
      if (vec) RVQ_EMBED(float, float, true); else RVQ_EMBED(float, float, false);
    }
  }
#undef RVQ_EMBED
  return hipGetLastError();
}

}  // namespace rvq
