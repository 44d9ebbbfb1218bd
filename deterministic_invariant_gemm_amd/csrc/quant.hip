// fp8 quantisation (AstrAI fp8_mm.cu: quantize_kernel, transpose_quantize_kernel
// and cast_fp8): every bf16 element times the inverse scale, multiplied in f32,
// converted to OCP e4m3fn or e5m2 with round-to-nearest-even, values beyond the
// largest finite one saturating to it (NaN stays NaN); the max-abs of the
// unscaled source is folded into *amax (NaN ignored).  The max of non-negative
// floats is the max of their bit patterns read as unsigned integers, so one
// atomic max per workgroup gives the same result in any order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace bi {

namespace {

constexpr int QT = 256;  // threads per workgroup
constexpr int64_t QCAP = 256;  // most workgroups of the quantiser (a grid-stride loop)

template <int FMT>
__device__ __forceinline__ float saturate(float v) {
    constexpr float M = FMT == DT_E5M2 ? 57344.0f : 448.0f;
    return v > M ? M : (v < -M ? -M : v);  // NaN: both tests false, passes through
}

// two f32 values -> two fp8 codes in bytes 0-1 (HI false) or 2-3 (HI true) of `old`
template <int FMT, bool HI>
__device__ __forceinline__ int cvt2(float a, float b, int old) {
    a = saturate<FMT>(a);
    b = saturate<FMT>(b);
    if constexpr (FMT == DT_E5M2) return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
    else return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

template <int FMT>
__device__ __forceinline__ uint8_t cvt1(float a) {
    return (uint8_t)(cvt2<FMT, false>(a, 0.0f, 0) & 0xff);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// max over the workgroup, then one atomic max on the bit pattern -- skipped
// when the value already in *amax is at least as large: the running max only
// grows, so such an atomic could not change it (a stale read only costs an
// unneeded atomic).  Thousands of workgroups each issuing an atomic on one
// address would otherwise serialise at the end of the kernel.
__device__ __forceinline__ void fold_amax(float mx, float *amax) {
    __shared__ float part[QT / 64];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = part[0];
#pragma unroll
        for (int w = 1; w < QT / 64; ++w) m = fmaxf(m, part[w]);
        unsigned int *bits = reinterpret_cast<unsigned int *>(amax);
        const unsigned int mb = __float_as_uint(m);
        if (mb > __hip_atomic_load(bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMax(bits, mb);
    }
}

// vec: src and dst 16-byte aligned.  Each thread converts UN chunks of 16
// elements per step (all loads issued first, so more bytes are in flight),
// the remainder element by element.  The source is read once (streaming
// loads); the codes are stored normally, so that the GEMM that reads them next
// finds them in the caches (streaming stores made the scaled linear 4-5 %
// slower).
constexpr int UN = 4;

template <int FMT>
__device__ __forceinline__ u32x4 convert16(const u32x4 a, const u32x4 b, float s, float &mx) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    int o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float f0 = lo_bf16(w[2 * q]), f1 = hi_bf16(w[2 * q]);
        const float f2 = lo_bf16(w[2 * q + 1]), f3 = hi_bf16(w[2 * q + 1]);
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(f0), fabsf(f1)), fmaxf(fabsf(f2), fabsf(f3))));
        o[q] = cvt2<FMT, true>(f2 * s, f3 * s, cvt2<FMT, false>(f0 * s, f1 * s, 0));
    }
    return u32x4{(uint32_t)o[0], (uint32_t)o[1], (uint32_t)o[2], (uint32_t)o[3]};
}

template <int FMT>
__global__ __launch_bounds__(QT) void quantize_kernel(const uint16_t *src, const float *scale_inv,
                                                      uint8_t *dst, float *amax, int64_t n,
                                                      int vec) {
    const float s = *scale_inv;
    float mx = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * QT;
    const int64_t tid = (int64_t)blockIdx.x * QT + threadIdx.x;
    int64_t done = 0;
    if (vec) {
        const int64_t nchunk = n / 16;
        const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
        u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
        int64_t c = tid;
        // full steps: chunks c, c + stride, ..., c + (UN-1) stride all exist
        for (; c + (UN - 1) * stride < nchunk; c += UN * stride) {
            u32x4 a[UN], b[UN];
#pragma unroll
            for (int u = 0; u < UN; ++u) {
                a[u] = __builtin_nontemporal_load(s4 + 2 * (c + u * stride));
                b[u] = __builtin_nontemporal_load(s4 + 2 * (c + u * stride) + 1);
            }
#pragma unroll
            for (int u = 0; u < UN; ++u)
                d4[c + u * stride] = convert16<FMT>(a[u], b[u], s, mx);
        }
        for (; c < nchunk; c += stride)
            d4[c] = convert16<FMT>(s4[2 * c], s4[2 * c + 1], s, mx);
        done = nchunk * 16;
    }
    for (int64_t i = done + tid; i < n; i += stride) {
        const float f = bf16_bits_to_f32(src[i]);
        mx = fmaxf(mx, fabsf(f));
        dst[i] = cvt1<FMT>(f * s);
    }
    if (amax) fold_amax(mx, amax);
}

// [rows, cols] -> [cols, rows] through a TR x 64 byte tile in LDS (TR source
// rows, 64 source columns): the source is read in 128-byte row pieces and the
// destination written in TR-byte row pieces.  vec_in: cols % 8 == 0 and src
// 16-byte aligned; vec_out: rows % 16 == 0 and dst 16-byte aligned.
constexpr int TR = 256;
// LDS layout of the tile: the dword holding source columns 4c .. 4c+3 of source
// row r sits at word r * TP + (c ^ tile_swz(r)).  With this pitch and swizzle
// the write phase's reads (lanes: 16 row blocks x 4 dword columns) fall in 64
// distinct banks and the read phase's writes meet at most two to a bank.
constexpr int TP = 19;
__device__ __forceinline__ int tile_swz(int r) { return 4 * ((r >> 6) & 3); }

// dst_rows (nullable): also the untransposed codes, [rows, cols], from the same
// read of the source; vec_rows: its 16-byte pieces may be stored whole.
template <int FMT>
__global__ __launch_bounds__(QT) void transpose_quantize_kernel(
    const uint16_t *src, const float *scale_inv, uint8_t *dst, uint8_t *dst_rows, float *amax,
    int64_t rows, int64_t cols, int vec_in, int vec_out, int vec_rows) {
    __shared__ uint32_t tile[TR][TP];
    const float s = *scale_inv;
    const int64_t r0 = (int64_t)blockIdx.y * TR, c0 = (int64_t)blockIdx.x * 64;
    const int t = threadIdx.x;
    float mx = 0.0f;
    // read: TR rows x 4 pieces of 16 columns; thread t takes rows t / 4 + 64 j
#pragma unroll
    for (int j = 0; j < TR / 64; ++j) {
        const int rr = (t >> 2) + 64 * j, cc = 16 * (t & 3);
        const int64_t gr = r0 + rr, gc = c0 + cc;
        float f[16];
        if (vec_in && gr < rows && gc + 16 <= cols) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(src + gr * cols + gc);
            const u32x4 a = p[0], b = p[1];
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int q = 0; q < 8; ++q) f[2 * q] = lo_bf16(w[q]), f[2 * q + 1] = hi_bf16(w[q]);
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q)
                f[q] = (gr < rows && gc + q < cols) ? bf16_bits_to_f32(src[gr * cols + gc + q])
                                                    : 0.0f;
        }
        uint32_t code[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(f[4 * q]), fabsf(f[4 * q + 1])),
                                 fmaxf(fabsf(f[4 * q + 2]), fabsf(f[4 * q + 3]))));
            code[q] = (uint32_t)cvt2<FMT, true>(
                f[4 * q + 2] * s, f[4 * q + 3] * s, cvt2<FMT, false>(f[4 * q] * s, f[4 * q + 1] * s, 0));
            tile[rr][(cc / 4 + q) ^ tile_swz(rr)] = code[q];
        }
        if (dst_rows && gr < rows) {
            uint8_t *d = dst_rows + gr * cols + gc;
            if (vec_rows && gc + 16 <= cols) {
                *reinterpret_cast<u32x4 *>(d) = u32x4{code[0], code[1], code[2], code[3]};
            } else {
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (gc + q < cols) d[q] = (uint8_t)((code[q >> 2] >> (8 * (q & 3))) & 0xffu);
            }
        }
    }
    __syncthreads();
    // write: thread t takes dword column c of the tile (destination rows
    // c0 + 4c .. c0 + 4c + 3) and source rows 16 rb .. 16 rb + 15 (16 bytes of
    // each of those destination rows): 16 LDS reads, a 4 x 4 byte transpose per
    // four of them, four 16-byte stores.  Lanes of a wave: rb = lane % 16,
    // c = lane / 16 + 4 * wave, so a store instruction writes 256 contiguous
    // bytes of each of four destination rows.
    static_assert(TR == 256 && QT == 256, "one thread per (row block, dword column)");
    {
        const int lane = t & 63, rb = lane & 15, c = (lane >> 4) + 4 * (t >> 6);
        uint32_t v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = tile[16 * rb + i][c ^ tile_swz(16 * rb + i)];
        // o[e][q]: bytes e of v[4q] .. v[4q+3], i.e. destination row 4c + e,
        // source rows 16 rb + 4q .. 16 rb + 4q + 3 (v_perm_b32 takes bytes 0-3
        // from its second operand, 4-7 from its first)
        uint32_t o[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t x = __builtin_amdgcn_perm(v[4 * q + 1], v[4 * q], 0x05010400u);
            const uint32_t y = __builtin_amdgcn_perm(v[4 * q + 1], v[4 * q], 0x07030602u);
            const uint32_t z = __builtin_amdgcn_perm(v[4 * q + 3], v[4 * q + 2], 0x05010400u);
            const uint32_t w = __builtin_amdgcn_perm(v[4 * q + 3], v[4 * q + 2], 0x07030602u);
            o[0][q] = __builtin_amdgcn_perm(z, x, 0x05040100u);
            o[1][q] = __builtin_amdgcn_perm(z, x, 0x07060302u);
            o[2][q] = __builtin_amdgcn_perm(w, y, 0x05040100u);
            o[3][q] = __builtin_amdgcn_perm(w, y, 0x07060302u);
        }
        const int64_t gr = r0 + 16 * rb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t go = c0 + 4 * c + e;
            if (go < cols && gr < rows) {
                uint8_t *d = dst + go * rows + gr;
                if (vec_out && gr + 16 <= rows) {
                    *reinterpret_cast<u32x4 *>(d) = u32x4{o[e][0], o[e][1], o[e][2], o[e][3]};
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (gr + i < rows) d[i] = (uint8_t)((o[e][i >> 2] >> (8 * (i & 3))) & 0xffu);
                }
            }
        }
    }
    if (amax) fold_amax(mx, amax);
}

__global__ void zero_kernel(float *a, float *b, float *c) {
    if (threadIdx.x == 0) {
        if (a) *a = 0.0f;
        if (b) *b = 0.0f;
        if (c) *c = 0.0f;
    }
}

}  // namespace

hipError_t launch_quantize(const void *src, const float *scale_inv, void *dst, float *amax,
                           int64_t n, int fmt, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int vec = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
    int64_t grid = (n / 16 + QT * UN - 1) / (QT * UN);
    if (grid < 1) grid = 1;
    // Fewer workgroups, fewer atomics on the one max-abs word: when that word
    // starts at zero (a fresh amax per call), nearly every workgroup's first
    // fold raises it, and those same-address atomics serialise.
    if (grid > QCAP) grid = QCAP;
    const uint16_t *sp = static_cast<const uint16_t *>(src);
    uint8_t *dp = static_cast<uint8_t *>(dst);
    if (fmt == DT_E5M2)
        hipLaunchKernelGGL(quantize_kernel<DT_E5M2>, dim3(grid), dim3(QT), 0, s, sp, scale_inv, dp,
                           amax, n, vec);
    else
        hipLaunchKernelGGL(quantize_kernel<DT_E4M3>, dim3(grid), dim3(QT), 0, s, sp, scale_inv, dp,
                           amax, n, vec);
    return hipGetLastError();
}

hipError_t launch_transpose_quantize(const void *src, const float *scale_inv, void *dst,
                                     void *dst_rows, float *amax, int64_t rows, int64_t cols,
                                     int fmt, hipStream_t s) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int64_t gx = (cols + 63) / 64, gy = (rows + TR - 1) / TR;
    if (gx > 0x7fffffffLL || gy > 65535) return hipErrorInvalidConfiguration;
    const int vec_in = cols % 8 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0;
    const int vec_out = rows % 16 == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
    const int vec_rows = cols % 16 == 0 && (reinterpret_cast<uintptr_t>(dst_rows) & 15) == 0;
    const uint16_t *sp = static_cast<const uint16_t *>(src);
    uint8_t *dp = static_cast<uint8_t *>(dst);
    uint8_t *rp = static_cast<uint8_t *>(dst_rows);
    if (fmt == DT_E5M2)
        hipLaunchKernelGGL(transpose_quantize_kernel<DT_E5M2>, dim3(gx, gy), dim3(QT), 0, s, sp,
                           scale_inv, dp, rp, amax, rows, cols, vec_in, vec_out, vec_rows);
    else
        hipLaunchKernelGGL(transpose_quantize_kernel<DT_E4M3>, dim3(gx, gy), dim3(QT), 0, s, sp,
                           scale_inv, dp, rp, amax, rows, cols, vec_in, vec_out, vec_rows);
    return hipGetLastError();
}

hipError_t launch_zero3(float *a, float *b, float *c, hipStream_t s) {
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, s, a, b, c);
    return hipGetLastError();
}

}  // namespace bi
