// Per-token top-k selection, gates and histogram counts, shared by the top-k
// kernel and the fused router + top-k kernel.
//
// Megatron-LM part 6, section "Router": top-k over the router scores picks
// each token's k experts, weighted by softmax or sigmoid.  infra-l7,
// "NVIDIA 原题": softmax over [T,E] and the top-k gate values; the
// DeepSeek-V3 bias only takes part in choosing the top-k.
#pragma once

#include "moe_device.h"

namespace moe {

template <int G>
__device__ __forceinline__ uint64_t seg_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) {
    const uint64_t o = __shfl_xor(v, m, G);
    v = o > v ? o : v;
  }
  return v;
}

// Selection key of expert e: ordered fp32 key bits << 32 | ~e, so that the
// largest key wins and equal keys go to the lower expert index.
__device__ __forceinline__ uint64_t topk_key(float key_value, int e) {
  return ((uint64_t)ordered_bits(key_value) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// One token per aligned segment of G lanes of a wave; lane s holds experts
// s, s+G, ... (NPL of them) with logits lg[] (-inf where absent) and keys
// key[] (0 where absent).  Each of the k rounds takes the segment maximum of
// the keys and the winner clears its entry; the winners are counted in the
// LDS histogram `hist` and written to sel_e/sel_l (this token's k LDS
// slots).  Then lanes s < k write the token's slot s: idx_row[s] and its
// gate gate_row[s] from the fp32 logits (never the selection bias):
//   gate_mode 0  softmax over the k selected
//   gate_mode 1  softmax over all E, at the selected experts
//   gate_mode 2  sigmoid, normalised over the k selected
// Every lane of the segment must call this (it shuffles across them).
template <int G, int NPL>
__device__ __forceinline__ void topk_segment(bool valid, int s, int E, int k, int gate_mode,
                                             const float (&lg)[NPL], uint64_t (&key)[NPL],
                                             int32_t* sel_e, float* sel_l, int32_t* hist,
                                             int32_t* idx_row, float* gate_row) {
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) best = key[i] > best ? key[i] : best;
    const uint64_t win = seg_max_u64<G>(best);
    if (win != 0) {
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        if (key[i] == win) {
          key[i] = 0;
          const int e = (int)(0xFFFFFFFFu - (uint32_t)win);
          sel_e[r] = e;
          sel_l[r] = lg[i];
          if (hist) atomicAdd(&hist[e], 1);
        }
      }
    }
  }
  // Segment lanes see the winners written by other lanes of the same wave.
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

  const bool slot = valid && s < k;
  const float l = slot ? sel_l[s] : -INFINITY;
  float g = 0.f;
  if (gate_mode == 0) {
    const float m = seg_max_f32<G>(l);
    const float num = slot ? expf(l - m) : 0.f;
    const float den = seg_sum_f32<G>(num);
    g = num / den;
  } else if (gate_mode == 1) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i) m = fmaxf(m, lg[i]);
    m = seg_max_f32<G>(m);
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) part += (s + G * i < E) ? expf(lg[i] - m) : 0.f;
    const float den = seg_sum_f32<G>(part);
    g = (slot ? expf(l - m) : 0.f) / den;
  } else {
    const float sg = slot ? 1.f / (1.f + expf(-l)) : 0.f;
    const float den = seg_sum_f32<G>(sg);
    g = sg / den;
  }
  if (slot) {
    idx_row[s] = sel_e[s];
    gate_row[s] = g;
  }
}

}  // namespace moe
