// Learned cluster representatives.
//
// AttentionIndex, paper-daily.com explainer, "代表向量为什么要学？": grouping stays
// by distance; a small network shared by the layer reads each new cluster's
// summaries (mean of the member keys, log of the size, mean and maximum over the
// members of a learned per-member transform) and adds a bounded correction to the
// mean.  It runs when a seal or a refit creates clusters; routing then scores the
// corrected representative like any other.
//
//   phi(x) = W2 ReLU(W1 x + b1) + b2                       (h = 128 hidden units)
//   z      = [mean, log n, mean_m phi(x_m), max_m phi(x_m)]
//   rep    = mean + alpha * tanh(Wb ReLU(Wa z + ba) + bb)
//
// Weights are packed fp32: W1 [h, d], b1 [h], W2 [h, h], b2 [h], Wa [h, d + 1 + 2h],
// ba [h], Wb [d, h], bb [d], alpha.  One block per cluster (blocks loop over
// clusters so the per-member weights are staged in LDS once per block).
#include "dispatch.h"
#include "launch.h"
#include "params.h"

namespace ivftk {

constexpr int ENC_H = 128;

__host__ __device__ constexpr int64_t enc_floats(int d) {
  return (int64_t)ENC_H * d + ENC_H + ENC_H * ENC_H + ENC_H + (int64_t)ENC_H * (d + 1 + 2 * ENC_H) + ENC_H +
         (int64_t)d * ENC_H + d + 1;
}

template <int DT, int D>
__global__ __launch_bounds__(256) void k_encode(EncParams p) {
  constexpr int H = ENC_H;
  __shared__ float w1t[D * H];      // w1t[i*H + j] = W1[j][i]
  __shared__ float w2t[H * H];      // w2t[k*H + j] = W2[j][k]
  __shared__ float xs[4][D];
  __shared__ float h1s[4][H];
  __shared__ float pmp[4][H], pxp[4][H];
  __shared__ float z[D + 1 + 2 * H];
  __shared__ float u[H];
  __shared__ uint32_t amax;
  const int tid = threadIdx.x, mi = tid >> 6, jj = tid & 63;
  const float* W1 = p.w;
  const float* b1 = W1 + H * D;
  const float* W2 = b1 + H;
  const float* b2 = W2 + H * H;
  const float* Wa = b2 + H;
  const float* ba = Wa + H * (D + 1 + 2 * H);
  const float* Wb = ba + H;
  const float* bb = Wb + D * H;
  const float alpha = bb[D];
  for (int e = tid; e < H * D; e += 256) w1t[(e % D) * H + e / D] = W1[e];
  for (int e = tid; e < H * H; e += 256) w2t[(e % H) * H + e / H] = W2[e];
  const int64_t nk1 = p.n_keys - 1;
  for (int b = blockIdx.x; b < p.n_slots; b += gridDim.x) {
    const int s = p.slot0 + b;
    const int n = p.st.size[s];
    const float* cent = p.st.cent + (size_t)s * D;
    float* out = p.lrep + (size_t)s * D;
    __syncthreads();   // weights staged; the previous cluster's readers are done
    if (n <= 0) {
      for (int i = tid; i < D; i += 256) out[i] = cent[i];
      continue;
    }
    const int* mem = p.st.members + max(p.st.off[s], 0);
    // ---- per-member transform, four members at a time; running mean/max per unit ----
    float sum0 = 0.0f, sum1 = 0.0f, mx0 = -__builtin_inff(), mx1 = -__builtin_inff();
    for (int g0 = 0; g0 < n; g0 += 4) {
      const int m = g0 + mi;
      const bool valid = m < n;
      {
        int64_t pos = mem[valid ? m : n - 1];
        pos = pos < 0 ? 0 : (pos > nk1 ? nk1 : pos);
        const uint8_t* row = p.keys + (size_t)pos * (D * Elem<DT>::bytes);
        const float sk = (DT == DT_E4M3) ? p.kscale[pos] : 1.0f;
        for (int i = jj; i < D; i += 64) {
          float v = load_elem<DT>(row, i);
          if constexpr (DT == DT_E4M3) v = v * sk;
          xs[mi][i] = v;
        }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int j = jj + 64 * q;
        float a = b1[j];
        for (int i = 0; i < D; ++i) a = a + w1t[i * H + j] * xs[mi][i];
        h1s[mi][j] = a > 0.0f ? a : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int j = jj + 64 * q;
        float f = b2[j];
        for (int k = 0; k < H; ++k) f = f + w2t[k * H + j] * h1s[mi][k];
        if (valid) {
          if (q == 0) {
            sum0 = sum0 + f;
            mx0 = __builtin_fmaxf(mx0, f);
          } else {
            sum1 = sum1 + f;
            mx1 = __builtin_fmaxf(mx1, f);
          }
        }
      }
      __syncthreads();   // xs and h1s are rewritten by the next group
    }
    pmp[mi][jj] = sum0;
    pmp[mi][jj + 64] = sum1;
    pxp[mi][jj] = mx0;
    pxp[mi][jj + 64] = mx1;
    if (tid == 0) amax = 0u;
    __syncthreads();
    // ---- summaries z = [mean, log n, pooled mean, pooled max] ----
    for (int i = tid; i < D; i += 256) z[i] = cent[i];
    if (tid == 0) z[D] = logf((float)n);
    if (tid < H) {
      const float sm = ((pmp[0][tid] + pmp[1][tid]) + pmp[2][tid]) + pmp[3][tid];
      z[D + 1 + tid] = sm / (float)n;
      z[D + 1 + H + tid] = __builtin_fmaxf(__builtin_fmaxf(pxp[0][tid], pxp[1][tid]),
                                           __builtin_fmaxf(pxp[2][tid], pxp[3][tid]));
    }
    __syncthreads();
    if (tid < H) {
      const float* wa = Wa + (size_t)tid * (D + 1 + 2 * H);
      float a = ba[tid];
      for (int i = 0; i < D + 1 + 2 * H; ++i) a = a + wa[i] * z[i];
      u[tid] = a > 0.0f ? a : 0.0f;
    }
    __syncthreads();
    // ---- corrected representative, then the key-format copy ----
    for (int i = tid; i < D; i += 256) {
      const float* wb = Wb + (size_t)i * H;
      float o = bb[i];
      for (int j = 0; j < H; ++j) o = o + wb[j] * u[j];
      const float r = cent[i] + alpha * tanhf(o);
      out[i] = r;
      if constexpr (DT == DT_F32) {
        reinterpret_cast<float*>(p.rep)[(size_t)s * D + i] = r;
      } else if constexpr (DT == DT_BF16) {
        reinterpret_cast<uint16_t*>(p.rep)[(size_t)s * D + i] = (uint16_t)f32_to_bf16(r);
      } else {
        atomicMax(&amax, __float_as_uint(__builtin_fabsf(r)));
      }
    }
    if constexpr (DT == DT_E4M3) {
      __syncthreads();
      const float am = __uint_as_float(amax);
      const float sr = am / 448.0f;
      for (int i = tid; i < D; i += 256)
        p.rep[(size_t)s * D + i] = (am == 0.0f) ? (uint8_t)0 : (uint8_t)f32_to_e4m3(out[i] / sr);
      if (tid == 0) p.rsc[s] = (am == 0.0f) ? 1.0f : sr;
    } else {
      if (tid == 0) p.rsc[s] = 1.0f;
    }
  }
}

template <int DT, int D>
static hipError_t launch_encode_t(const EncParams& p, hipStream_t s) {
  if (p.n_slots <= 0) return hipSuccess;
  int dev = 0, n_cu = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  const int grid = p.n_slots < n_cu ? p.n_slots : n_cu;
  hipLaunchKernelGGL((k_encode<DT, D>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_encode(const EncParams& p, int dtype, int dim, hipStream_t s) {
  IVFTK_DISPATCH_D(launch_encode_t, dtype, dim, p, s);
}

int64_t encoder_floats(int dim) { return enc_floats(dim); }

}  // namespace ivftk
