// Sliding-window branch: the last 128 tokens of each sequence in FP8, and
// their attention merged with the sparse branch, for gfx950.
//
// What is computed ("Le cache KV en FP4 — les 890 octets, vérifiés", section
// "La contrepartie : la fenêtre glissante": a per-layer window in FP8 of
// 512 + 512/16 bytes per token; "DeepSeek V4.1 Flash : 890 octets de cache KV
// par token", section "L'architecture : trois leviers contre le cache": the
// window is 128 tokens). A token's window row is its 512-channel latent: 512
// E4M3FN bytes (channel c at byte c) then one E8M0 scale byte per 16 channels,
// the smallest power of two 2^X with amax <= 448 * 2^X (no value saturates);
// values are E4M3FN nearest-even of x * 2^-X. The ring holds token t in row
// t mod 128. The window's attention (same heads, same tau) and the sparse
// branch's (o, lse) merge into one softmax over the union of both sets:
// o = (e^lse_s o_s + e^lse_w o_w) / (e^lse_s + e^lse_w).
//
// swa_write_kernel      16 tokens x 16 lanes per workgroup; a lane packs 32
//                       channels (two scale blocks) with 16-byte loads/stores.
// swa_attention_kernel  workgroup = (sequence, 16 heads), 8 waves. Wave w
//                       dequantizes window tile w (16 tokens) to bf16 with
//                       the scaled FP8 conversion (an E4M3 value times a
//                       power of two is exact in bf16),
//                       contracts QK^T with v_mfma_f32_16x16x32_bf16 straight
//                       from registers, and stores the tile in LDS; the
//                       workgroup takes the softmax per head; then wave w
//                       owns 64 latent dims and contracts O^T = C^T P^T over
//                       the 128 tokens, C^T read with the transposing LDS
//                       read and P split into two bf16 terms (hi + lo) so the
//                       weights keep 16 bits; finally each lane merges its
//                       outputs with the sparse branch's through the two lse.
#include "device.h"
#include "codec_dev.h"
#include "kernels.h"
#include <atomic>
#include <math.h>

namespace csa2 {

constexpr int SW_WIN = kSwaWindow;            // 128 tokens
constexpr int SW_ROW = kSwaRowBytes;          // 544 bytes
constexpr int SW_PITCH = 1056;                // bytes per bf16 token row in LDS (rows 8 banks apart)
constexpr int SW_SLOT = 16 * SW_PITCH;        // one tile of 16 tokens
constexpr int SW_LDS = 8 * SW_SLOT;           // 135168: the whole window
constexpr int SW_THREADS = 512;

// E8M0 exponent X of a block: the smallest X with amax <= 448 * 2^X (amax > 0),
// clamped to [-127, 127]; exact (binary exponent, power-of-two scaling).
__device__ __forceinline__ int window_block_exponent(float amax) {
  const int x0 = floor_log2(amax) - 8;        // amax * 2^-x0 in [256, 512)
  int x = ldexpf(amax, -x0) > 448.0f ? x0 + 1 : x0;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// grid (ceil(min(T, 128) / 16), B): tokens T - min(T, 128) .. T - 1 of each
// sequence (earlier ones would be overwritten in the ring anyway).
__global__ __launch_bounds__(256) void swa_write_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                        const int64_t* __restrict__ pos0,
                                                        uint8_t* __restrict__ win) {
  const int b = blockIdx.y, tid = threadIdx.x;
  const int64_t tw = T < SW_WIN ? T : SW_WIN;
  const int64_t tl = (int64_t)blockIdx.x * 16 + (tid >> 4);
  if (tl >= tw) return;
  const int64_t t = T - tw + tl;
  const int p = tid & 15;                      // channels 32p .. 32p + 31: blocks 2p, 2p + 1
  const uint16_t* src = x + ((int64_t)b * T + t) * 512 + 32 * p;
  u32x4_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = *(const u32x4_t*)(src + 8 * i);
  const int64_t row = (pos0[b] + t) & (SW_WIN - 1);
  uint8_t* dst = win + ((int64_t)b * SW_WIN + row) * SW_ROW;
  uint32_t sbytes = 0;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    float xv[16], amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t d = v[2 * blk + (i >> 2)][i & 3];
      xv[2 * i] = bf16_to_f32(d & 0xFFFFu);
      xv[2 * i + 1] = bf16_to_f32(d >> 16);
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(xv[c]));
    u32x4_t out = {0, 0, 0, 0};
    uint32_t sb = 0;
    if (amax > 0.0f) {
      const int X = window_block_exponent(amax);
      sb = (uint32_t)(X + 127);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        float val;
        const uint32_t code = e4m3fn_rne(ldexpf(fabsf(xv[c]), -X), &val) | ((__float_as_uint(xv[c]) >> 24) & 0x80u);
        out[c >> 2] |= code << (8 * (c & 3));
      }
    }
    *(u32x4_t*)(dst + 32 * p + 16 * blk) = out;
    sbytes |= sb << (8 * blk);
  }
  *(uint16_t*)(dst + 512 + 2 * p) = (uint16_t)sbytes;
}

__global__ __launch_bounds__(SW_THREADS) void swa_attention_kernel(
    const uint8_t* __restrict__ win, const int32_t* __restrict__ n_win, const uint16_t* __restrict__ q, int H,
    float tau, float* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // the bf16 window, tile w in slot w
  __shared__ float lg[SW_WIN][17];             // logits, then the weights e^(l - max); [token][head]
  __shared__ float lse_w[16], inv_w[16];
  const int HG = (H + 15) / 16;
  const int b = blockIdx.x / HG, hg = blockIdx.x % HG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, kg = lane >> 4;
  const int nw = min(max(n_win[b], 0), SW_WIN);

  // --- QK: wave w takes tokens 16w .. 16w + 15; lane (r, kg) holds token 16w + r,
  // dims 128kg .. 128kg + 127, and the query of head 16hg + r on the same dims
  const int head_q = 16 * hg + r;
  bf16x8_t qb[16];
  {
    const uint16_t* qr = q + ((int64_t)b * H + (head_q < H ? head_q : 0)) * 512 + 128 * kg;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      u32x4_t v = *(const u32x4_t*)(qr + 8 * j);
      if (head_q >= H) v = u32x4_t{0, 0, 0, 0};
      __builtin_memcpy(&qb[j], &v, 16);
    }
  }
  // the sparse branch's result this lane merges into, requested up front:
  // dims 64w + 16u + 4kg .. +3 of head 16hg + r (see the merge below)
  const int head = 16 * hg + r;
  const bool head_ok = head < H;
  float* ob = out + ((int64_t)b * H + (head_ok ? head : 0)) * 512 + 64 * wave + 4 * kg;
  float4 os[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) os[u] = *(const float4*)(ob + 16 * u);
  const float ls = lse[(int64_t)b * H + (head_ok ? head : 0)];
  const int tok = 16 * wave + r;
  const bool tok_ok = tok < nw;
  const uint8_t* wrow = win + ((int64_t)b * SW_WIN + (tok_ok ? tok : 0)) * SW_ROW;
  u32x4_t cw[8];
  u32x2_t sw;
#pragma unroll
  for (int c = 0; c < 8; ++c) cw[c] = *(const u32x4_t*)(wrow + 128 * kg + 16 * c);
  sw = *(const u32x2_t*)(wrow + 512 + 8 * kg);
  if (!tok_ok) {
#pragma unroll
    for (int c = 0; c < 8; ++c) cw[c] = u32x4_t{0, 0, 0, 0};
    sw = u32x2_t{0, 0};
  }
  uint8_t* slot = smem + wave * SW_SLOT + r * SW_PITCH + 256 * kg;
  f32x4_t acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {            // dims 128kg + 8jj .. +7: block 8kg + jj/2
    const uint32_t sbyte = (sw[jj >> 3] >> (8 * ((jj >> 1) & 3))) & 0xFFu;
    const float scale = __uint_as_float(sbyte << 23);   // 2^(sbyte - 127); byte 0 holds zeros only
    const uint32_t w0 = cw[jj >> 1][2 * (jj & 1)], w1 = cw[jj >> 1][2 * (jj & 1) + 1];
    // gfx950's scaled FP8 (E4M3FN) -> bf16 conversion applies the power of two exactly
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false);
    const bf16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true);
    const bf16x8_t ca = {a[0], a[1], c[0], c[1], d[0], d[1], e[0], e[1]};
    u32x4_t pk;
    __builtin_memcpy(&pk, &ca, 16);
    acc[jj & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca, qb[jj], acc[jj & 1], 0, 0, 0);
    *(u32x4_t*)(slot + 16 * jj) = pk;
  }
  {
    const f32x4_t l4 = acc[0] + acc[1];          // tokens 16w + 4kg + i, head r
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * wave + 4 * kg + i;
      lg[t][r] = t < nw ? tau * l4[i] : -INFINITY;
    }
  }
  __syncthreads();

  // --- softmax per head: 32 threads per head, 4 tokens each
  {
    const int h = tid >> 5, j = tid & 31;
    float l[4], m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) { l[i] = lg[4 * j + i][h]; m = fmaxf(m, l[i]); }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = l[i] == -INFINITY ? 0.0f : expf(l[i] - m);
      lg[4 * j + i][h] = pv;
      s += pv;
    }
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) s += __shfl_xor(s, o, 32);
    if (j == 0) {
      lse_w[h] = s > 0.0f ? m + logf(s) : -INFINITY;
      inv_w[h] = s > 0.0f ? 1.0f / s : 0.0f;
    }
  }
  __syncthreads();

  // --- PV: wave w owns dims 64w .. 64w + 63 (4 tiles of 16); K steps over the
  // slot pairs (2k, 2k + 1); lane i of group kg reads dim 16u + i of tokens
  // 4kg .. 4kg + 3 of a slot with the transposing read
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const int toff = (4 * kg + (r >> 2)) * SW_PITCH + 8 * (r & 3) + 2 * 64 * wave;
  f32x4_t O[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) O[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int s0 = 2 * k, s1 = 2 * k + 1;
    // B: weights of tokens 16 s0 + 4kg + i (K 0..3) and 16 s1 + 4kg + i (K 4..7), head r
    float pw[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = lg[16 * s0 + 4 * kg + i][r];
      pw[4 + i] = lg[16 * s1 + 4 * kg + i][r];
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a0 = __float_as_uint(pw[2 * i]) & 0xFFFF0000u, a1 = __float_as_uint(pw[2 * i + 1]) & 0xFFFF0000u;
      const float r0 = pw[2 * i] - __uint_as_float(a0), r1 = pw[2 * i + 1] - __uint_as_float(a1);
      hi[i] = (a0 >> 16) | a1;
      lo[i] = ((__float_as_uint(r0) + 0x7FFFu + ((__float_as_uint(r0) >> 16) & 1u)) >> 16) |
              ((__float_as_uint(r1) + 0x7FFFu + ((__float_as_uint(r1) >> 16) & 1u)) & 0xFFFF0000u);
    }
    bf16x8_t bh, bl;
    __builtin_memcpy(&bh, hi, 16);
    __builtin_memcpy(&bl, lo, 16);
    __attribute__((address_space(3))) uint8_t* base = (__attribute__((address_space(3))) uint8_t*)smem;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const i16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + s0 * SW_SLOT + toff + 32 * u));
      const i16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + s1 * SW_SLOT + toff + 32 * u));
      bf16x8_t a;
      __builtin_memcpy(&a, &a0, 8);
      __builtin_memcpy((uint8_t*)&a + 8, &a1, 8);
      O[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, O[u], 0, 0, 0);
      O[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, O[u], 0, 0, 0);
    }
  }

  // --- merge with the sparse branch: lane (r, kg) holds dims 64w + 16u + 4kg + i of head r
  if (!head_ok) return;
  const float lw = lse_w[r], iw = inv_w[r];
  const float mm = fmaxf(ls, lw);
  const float a_s = ls == -INFINITY ? 0.0f : expf(ls - mm);
  const float a_w = lw == -INFINITY ? 0.0f : expf(lw - mm);
  const float z = a_s + a_w;
  const float f_s = z > 0.0f ? a_s / z : 0.0f, f_w = z > 0.0f ? a_w * iw / z : 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const f32x4_t ow = O[u];
    *(float4*)(ob + 16 * u) = float4{f_s * os[u].x + f_w * ow[0], f_s * os[u].y + f_w * ow[1],
                                     f_s * os[u].z + f_w * ow[2], f_s * os[u].w + f_w * ow[3]};
  }
  if (wave == 0 && kg == 0) lse[(int64_t)b * H + head] = z > 0.0f ? mm + logf(z) : -INFINITY;
}

hipError_t launch_swa_write(const uint16_t* x, int B, int64_t T, const int64_t* pos0, uint8_t* win,
                            hipStream_t stream) {
  const int64_t tw = T < SW_WIN ? T : SW_WIN;
  if (tw <= 0) return hipSuccess;
  dim3 grid((unsigned)((tw + 15) / 16), (unsigned)B), block(256);
  hipLaunchKernelGGL(swa_write_kernel, grid, block, 0, stream, x, T, pos0, win);
  return hipGetLastError();
}

hipError_t launch_swa_attention(const uint8_t* win, const int32_t* n_win, const uint16_t* q, int B, int H,
                                float tau, float* out, float* lse, hipStream_t stream) {
  static std::atomic<uint32_t> attr_set[64];
  int dev = 0;
  hipError_t e0 = hipGetDevice(&dev);
  if (e0 != hipSuccess) return e0;
  if (dev < 0 || dev >= 64 || !attr_set[dev].load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute((const void*)swa_attention_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SW_LDS);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_set[dev].store(1u, std::memory_order_release);
  }
  dim3 grid((unsigned)(B * ((H + 15) / 16))), block(SW_THREADS);
  hipLaunchKernelGGL(swa_attention_kernel, grid, block, SW_LDS, stream, win, n_win, q, H, tau, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
