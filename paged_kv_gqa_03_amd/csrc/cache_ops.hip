// cache_ops.hip -- the cache writes and the rotation that precede attention,
// for gfx950: paged KV append, fp8 quantize-on-write of sliding-window cache
// rows, and rotary embedding.  All three are HBM-bound streams of 16-byte
// vector loads and stores.
//
// Method:
//   - paged KV append (AstrAI "CUDA Kernels" doc, Backend Layer: the
//     attention backend owns the KV cache writes that precede paged decode
//     and prefill): new token i of sequence b lands at position
//     start_pos[b] + i, i.e. page bt[b][pos / ps], slot pos % ps;
//   - fp8 quantize-on-write (native_swa_decode.py: the cache holds OCP
//     e4m3fn codes plus a per-slot inverse scale; AstrAI doc, FP8 section:
//     quantize takes the multiplier and multiplies by it, amax is reported
//     in the input domain): code = e4m3fn(x * m) rounded to nearest even and
//     saturated at 448, the product taken in binary32; the slot's inverse
//     scale is bf16(1 / m); m = 448 / amax when the caller gives none;
//   - rotary (AstrAI doc, Rotary Embedding Kernel and Rotary Backend): the
//     cos / sin rows of the token's position are looked up in fp32 tables
//     and each adjacent pair (x[2i], x[2i+1]) is multiplied, as a complex
//     number, by cos_i + i sin_i; the math is fp32 and the result is rounded
//     to bf16 once.
#include "device_common.hpp"
#include "kernels.hpp"

namespace pa {

namespace {

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

// ------------------------------------------------------------ KV append

// One workgroup per new row.  The row's sequence b is the first with
// indptr[b + 1] > i, found 64 sequences at a time by one round of vector
// loads and a ballot; the same round brings indptr[b] and start_pos[b], so
// the row's page lookup waits for a single dependent load instead of a
// binary search's log2(B).
__global__ __launch_bounds__(256) void kv_append_kernel(const KvAppendParams p) {
    const int i = blockIdx.x;
    const int lane = threadIdx.x & 63;
    int b = p.B, first = 0, start = 0;
    for (int base = 0; base < p.B; base += 64) {
        const int k = base + lane;
        const bool in = k < p.B;
        const int hi = in ? p.indptr[k + 1] : 0;
        const int lo = in ? p.indptr[k] : 0;
        const int sp = in ? p.start_pos[k] : 0;
        const uint64_t hit = __ballot(in && hi > i);
        if (hit) {
            const int l = __ffsll((unsigned long long)hit) - 1;
            b = base + l;
            first = __shfl(lo, l);
            start = __shfl(sp, l);
            break;
        }
    }
    if (b >= p.B) return;
    const int64_t pos = (int64_t)start + (i - first);
    if (pos < 0) return;
    const int32_t page = p.bt[(int64_t)b * p.bt_sb + pos / p.ps];
    if (page < 0 || page >= p.num_pages) return;   // not a page of the pool: nothing is written
    const int64_t base = (int64_t)page * p.s_page + (pos % p.ps) * p.s_slot;
    const int cpr = p.D / 8;                         // 16-byte chunks per head row
    const int C = p.Hkv * cpr;                        // chunks per tensor row
    for (int c = threadIdx.x; c < 2 * C; c += blockDim.x) {
        const bool is_v = c >= C;
        const int cc = is_v ? c - C : c;
        const int g = cc / cpr, d = (cc - g * cpr) * 8;
        const uint16_t *src = (is_v ? p.v_new : p.k_new) + (int64_t)i * p.n_st + (int64_t)g * p.n_sh + d;
        uint16_t *dst = (is_v ? p.v_pool : p.k_pool) + base + (int64_t)g * p.s_head + d;
        st16(dst, ld16(src));
    }
}

// ------------------------------------------------- fp8 quantize-on-write

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)(u >> 16);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// One wave per row of HD = 512: lane l holds elements 8l .. 8l+7.
__global__ __launch_bounds__(256) void swa_quantize_kernel(const SwaQuantParams p) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= p.N) return;
    const uint4 raw = ld16(p.x + (int64_t)n * p.x_st + 8 * lane);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = bf16_lo(w[k]);
        v[2 * k + 1] = bf16_hi(w[k]);
    }
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s));
    const float m = p.mult ? p.mult[n] : (amax > 0.f ? 448.0f / amax : 1.0f);
    if (lane == 0 && p.amax) p.amax[n] = amax;
    const int64_t slot = p.slots[n];
    if (slot < 0 || slot >= p.num_slots) return;   // not a slot of the cache: nothing is written
    const uint32_t blk = divu32((uint32_t)slot, p.bs_div);
    const uint32_t off = (uint32_t)slot - blk * (uint32_t)p.bs;
    // Codes from the hardware conversion (v_cvt_pk_fp8_f32: nearest even,
    // OCP e4m3fn on gfx950).  Checked against the format's definition on
    // every code, every midpoint between neighbouring codes and its two
    // neighbouring floats, subnormals and signed zeros: bit-exact, except
    // that the conversion turns overflow and infinities into NaN and keeps
    // a NaN's sign.  So magnitudes are clamped to 448 first (saturation), and
    // NaN products give 0x7F through a byte mask.
    float y[8];
    uint32_t nan_lo = 0, nan_hi = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float t = v[k] * m;   // the product in binary32
        const uint32_t nm = (t != t) ? (0xffu << (8 * (k & 3))) : 0u;
        if (k < 4) nan_lo |= nm;
        else nan_hi |= nm;
        y[k] = fminf(fmaxf(t, -448.0f), 448.0f);
    }
    uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)lo, true);
    uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)hi, true);
    lo = (lo & ~nan_lo) | (0x7f7f7f7fu & nan_lo);
    hi = (hi & ~nan_hi) | (0x7f7f7f7fu & nan_hi);
    *reinterpret_cast<uint2 *>(p.cache + (int64_t)blk * p.c_sb + (int64_t)off * p.c_ss + 8 * lane) =
        make_uint2(lo, hi);
    if (lane == 0) p.inv_scale[slot * p.s_ss] = bf16_rne(1.0f / m);
}

// ------------------------------------------------------------- rotary

// One row of workgroups per token (blockIdx.x): its H head rows of D/8
// 16-byte chunks (four pairs each) are spread over blockIdx.y and the
// threads, so the token's position is one uniform load and the index math
// stays 32-bit.
__global__ __launch_bounds__(256) void rotary_kernel(const RotaryParams p) {
    const int cpr = p.D / 8;
    const int t = blockIdx.x;
    const int j = blockIdx.y * blockDim.x + threadIdx.x;   // chunk among the token's H rows
    if (j >= p.H * cpr) return;
    const int h = j / cpr, c = j - h * cpr;
    // The row's chunk goes out with the position load, not after it.
    const uint4 raw = ld16(p.x + (int64_t)t * p.x_st + (int64_t)h * p.x_sh + 8 * c);
    const int pos = p.pos[t];
    if (pos < 0 || pos >= p.rows) return;          // outside the table: the row is left as it is
    const float4 cs = *reinterpret_cast<const float4 *>(p.cos + (int64_t)pos * p.tab_st + 4 * c);
    const float4 sn = *reinterpret_cast<const float4 *>(p.sin + (int64_t)pos * p.tab_st + 4 * c);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    const float cv[4] = {cs.x, cs.y, cs.z, cs.w}, sv[4] = {sn.x, sn.y, sn.z, sn.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float a = bf16_lo(w[k]), b = bf16_hi(w[k]);
        const float re = fmaf(a, cv[k], -b * sv[k]);
        const float im = fmaf(a, sv[k], b * cv[k]);
        o[k] = (uint32_t)bf16_rne(re) | ((uint32_t)bf16_rne(im) << 16);
    }
    st16(p.out + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + 8 * c, make_uint4(o[0], o[1], o[2], o[3]));
}

}  // namespace

hipError_t launch_kv_append(const KvAppendParams &p, hipStream_t stream) {
    if (p.N <= 0) return hipSuccess;
    hipLaunchKernelGGL(kv_append_kernel, dim3(p.N), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_swa_quantize(const SwaQuantParams &p, hipStream_t stream) {
    if (p.N <= 0) return hipSuccess;
    hipLaunchKernelGGL(swa_quantize_kernel, dim3((p.N + 3) / 4), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_rotary(const RotaryParams &p, hipStream_t stream) {
    const int per_token = p.H * (p.D / 8);   // 16-byte chunks of one token
    if (p.T <= 0 || per_token <= 0) return hipSuccess;
    const int threads = per_token >= 256 ? 256 : (per_token + 63) / 64 * 64;
    const int ny = (per_token + threads - 1) / threads;
    if (ny > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rotary_kernel, dim3((unsigned)p.T, (unsigned)ny), dim3(threads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
