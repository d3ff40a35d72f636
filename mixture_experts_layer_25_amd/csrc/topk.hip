// Top-k selection, gates and the per-chunk expert histogram.
//
// Megatron-LM part 6, section "Router": top-k over the router scores picks
// each token's k experts, weighted by softmax or sigmoid.  infra-l7,
// "NVIDIA 原题": softmax over [T,E] and the top-k gate values; the
// DeepSeek-V3 bias only takes part in choosing the top-k.
//
// A token is handled by a segment of G lanes of one wave (G = the next
// power of two >= E up to 64 experts, 16 for 65..256 experts so that a
// wave takes 4 tokens at a time with 4-step shuffles, else 64); lane s of
// the segment holds experts s, s+G, s+2G, ...  Each of the k rounds takes
// the segment maximum of a
// 64-bit key (ordered fp32 key bits << 32 | ~expert), so the largest key
// wins and equal keys go to the lower expert index; the winner clears its
// entry.  Gates use the fp32 logits (never the selection bias).  Each
// workgroup covers 4 passes of 256/G tokens (one pass of 16 tokens with
// 16-lane segments) and writes the expert histogram of those tokens, which
// the scan kernel turns into ranks and offsets.
#include "moe_device.h"
#include "moe_internal.h"
#include "topk_device.h"

namespace moe {

namespace {

template <int G, int NPL, int PASSES>
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ sbias,
    int gate_mode, int64_t T, int E, int k, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, int32_t* __restrict__ chunk_hist) {
  constexpr int kTokPerPass = 256 / G;
  constexpr int kPasses = PASSES;
  constexpr int kTok = kPasses * kTokPerPass;
  __shared__ int32_t hist[1024];
  __shared__ int32_t sel_e[kTok][16];
  __shared__ float sel_l[kTok][16];

  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();

  const int seg = tid / G;           // token slot within a pass
  const int s = tid % G;             // lane within the segment
  const int64_t chunk0 = (int64_t)blockIdx.x * kTok;

  for (int pass = 0; pass < kPasses; ++pass) {
    const int tl = pass * kTokPerPass + seg;   // token within the chunk
    const int64_t t = chunk0 + tl;
    const bool valid = t < T;
    uint64_t key[NPL];
    float lg[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = s + G * i;
      key[i] = 0;
      lg[i] = -INFINITY;
      if (valid && e < E) {
        const float l = logits[t * E + e];
        lg[i] = l;
        key[i] = topk_key(sbias ? l + sbias[e] : l, e);
      }
    }
    topk_segment<G, NPL>(valid, s, E, k, gate_mode, lg, key, sel_e[tl], sel_l[tl], hist,
                         idx_out + t * k, gate_out + t * k);
  }
  if (chunk_hist) {
    __syncthreads();
    for (int e = tid; e < E; e += 256) chunk_hist[blockIdx.x * (int64_t)E + e] = hist[e];
  }
}

template <int G, int NPL, int PASSES = 4>
void launch_topk_t(const float* logits, const float* sb, int gate, int64_t T,
                   int E, int k, int32_t* idx, float* g, int32_t* hist,
                   hipStream_t s) {
  constexpr int tok = PASSES * (256 / G);
  const int64_t nwg = (T + tok - 1) / tok;
  MOE_LAUNCH((topk_kernel<G, NPL, PASSES>), dim3((unsigned)nwg), dim3(256), 0,
                     s, logits, sb, gate, T, E, k, idx, g, hist);
}

}  // namespace

hipError_t launch_topk(const float* logits, const float* select_bias, int gate,
                       int64_t T, int E, int k, int32_t* idx, float* gate_out,
                       int32_t* chunk_hist, hipStream_t s) {
  // G and the tokens per workgroup must agree with topk_kernel_tokens(E)
  if (E <= 8)
    launch_topk_t<8, 1>(logits, select_bias, gate, T, E, k, idx, gate_out, chunk_hist, s);
  else if (E <= 16)
    launch_topk_t<16, 1>(logits, select_bias, gate, T, E, k, idx, gate_out, chunk_hist, s);
  else if (E <= 32)
    launch_topk_t<32, 1>(logits, select_bias, gate, T, E, k, idx, gate_out, chunk_hist, s);
  else if (E <= 64)
    launch_topk_t<64, 1>(logits, select_bias, gate, T, E, k, idx, gate_out, chunk_hist, s);
  else if (E <= 128)
    launch_topk_t<16, 8, 1>(logits, select_bias, gate, T, E, k, idx, gate_out, chunk_hist, s);
  else if (E <= 256)
    launch_topk_t<16, 16, 1>(logits, select_bias, gate, T, E, k, idx, gate_out, chunk_hist, s);
  else if (E <= 512)
    launch_topk_t<64, 8>(logits, select_bias, gate, T, E, k, idx, gate_out, chunk_hist, s);
  else
    launch_topk_t<64, 16>(logits, select_bias, gate, T, E, k, idx, gate_out, chunk_hist, s);
  return hipGetLastError();
}

}  // namespace moe
