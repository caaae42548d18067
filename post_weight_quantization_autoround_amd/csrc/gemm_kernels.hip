// MFMA GEMMs of the tuning loop (gfx950).
//
// Both GEMMs of a step (blog sec. 3 algorithm flow: the QDQ forward and the
// back-propagation) are written as C[i, j] = sum_r A[i, r] * B[j, r] with
// both operands contiguous along the reduction index r:
//   forward  Y[m, n]  = sum_k X_b[m, k] * w^[n, k]     (A = X_b, B = w^)
//   wgrad    G[n, k]  = sum_m dY^T[n, m] * X_b^T[k, m] (A = dY^T, B = X_b^T)
// The forward epilogue writes dY^T directly and the calibration pool is kept
// transposed per sample ([S, K, T]) in HBM, so neither GEMM needs a transpose
// in LDS.  Rows of X_b (forward) and reduction columns of X_b^T (wgrad) are
// gathered from the pool by a per-step sample table in device memory, so one
// captured launch serves every step.
//
// Tiling: a workgroup computes a BM x BN tile with 64-wide wavefronts each
// owning a WM x WN sub-tile made of 32 x 32 MFMA blocks with fp32
// accumulators.  Operand tiles of BK reduction elements are staged through
// LDS (double buffered, one barrier per BK step): global loads for the next
// stage are issued before the MFMAs of the current one.  Rows in LDS are
// padded by 16 bytes so the 16-byte fragment reads of 32 consecutive rows hit
// distinct banks.  Workgroups are remapped so consecutive tiles land on the
// same XCD (dispatch is round-robin over the 8 XCDs) and share its L2.
#include "ar_internal.h"

namespace ar {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

struct SchedView {
    const int32_t* ids;  // NULL: identity
    __device__ __forceinline__ int64_t id(int64_t s) const { return ids ? (int64_t)ids[s] : s; }
};

__device__ __forceinline__ SchedView sched_view(const GemmArgs& a) {
    SchedView v;
    v.ids = nullptr;
    if (a.sched) {
        int64_t row = 0;
        if (a.state) row = a.after_decide ? a.state->t_eval : a.state->step;
        v.ids = a.sched + row * a.nseg;
    }
    return v;
}

// Element offset of row `i` of an operand (column part added separately).
__device__ __forceinline__ int64_t row_offset(const Operand& op, const SchedView& sv, int64_t i) {
    if (op.seg_len > 0 && !op.seg_cols) {
        const int64_t seg = i / op.seg_len;
        return sv.id(seg) * op.seg_stride + (i - seg * op.seg_len) * op.ld;
    }
    return i * op.ld;
}

// Element offset of reduction column k0 (start of a BK tile; a tile never
// crosses a segment because BK divides the segment length).
__device__ __forceinline__ int64_t col_offset(const Operand& op, const SchedView& sv, int64_t k0) {
    if (op.seg_len > 0 && op.seg_cols) {
        const int64_t seg = k0 / op.seg_len;
        return sv.id(seg) * op.seg_stride + (k0 - seg * op.seg_len);
    }
    return k0;
}

__device__ __forceinline__ int remap_block() {
    const int nb = gridDim.x, b = blockIdx.x;
    const int full = nb & ~7;
    return b < full ? (b & 7) * (full >> 3) + (b >> 3) : b;
}

// Epilogue over the accumulators of one wavefront.  Accumulator r of the
// 32 x 32 block (tm, tn) holds element
//   row 8*(r/4) + 4*(lane/32) + r%4,  column lane%32.
template <int TM, int TN, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& a, const SchedView& sv, floatx16 (&acc)[TM][TN],
                                         int64_t row0, int64_t col0, int lane, double* red) {
    const int half = lane >> 5;
    const int cl = lane & 31;
    float lsum = 0.0f;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int64_t j = col0 + tn * 32 + cl;
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int64_t i0 = row0 + tm * 32 + rg * 8 + half * 4;
                if (EPI == EPI_STORE) {
                    if (j < a.J) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (i0 + e < a.I) a.out[(i0 + e) * a.ldc + j] = acc[tm][tn][rg * 4 + e];
                    }
                } else {
                    float d[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t i = i0 + e;
                        d[e] = 0.0f;
                        if (i < a.I && j < a.J) {
                            const int64_t seg = i / a.yref_T;
                            const int64_t prow = sv.id(seg) * a.yref_T + (i - seg * a.yref_T);
                            d[e] = acc[tm][tn][rg * 4 + e] - a.yref[prow * a.yref_ld + j];
                            lsum += d[e] * d[e];
                        }
                    }
                    if (j < a.J) {
                        if (i0 + 3 < a.I) {
                            if (a.dyt_bf16) {
                                uint2 o;
                                o.x = (uint32_t)f32_to_bf16(a.dscale * d[0]) | ((uint32_t)f32_to_bf16(a.dscale * d[1]) << 16);
                                o.y = (uint32_t)f32_to_bf16(a.dscale * d[2]) | ((uint32_t)f32_to_bf16(a.dscale * d[3]) << 16);
                                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dyt) + j * a.lddyt + i0) = o;
                            } else {
                                *reinterpret_cast<float4*>(static_cast<float*>(a.dyt) + j * a.lddyt + i0) =
                                    make_float4(a.dscale * d[0], a.dscale * d[1], a.dscale * d[2], a.dscale * d[3]);
                            }
                        } else {
                            for (int e = 0; e < 4; ++e) {
                                if (i0 + e < a.I) {
                                    if (a.dyt_bf16)
                                        static_cast<uint16_t*>(a.dyt)[j * a.lddyt + i0 + e] = f32_to_bf16(a.dscale * d[e]);
                                    else
                                        static_cast<float*>(a.dyt)[j * a.lddyt + i0 + e] = a.dscale * d[e];
                                }
                            }
                        }
                    }
                }
            }
        }
    }
    if (EPI == EPI_LOSS) {
        double v = (double)lsum;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) red[threadIdx.x >> 6] = v;
    }
}

// ------------------------------------------------------------------ bf16 --
template <int BM, int BN, int BK, int WM, int WN, int EPI>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64) gemm_bf16_kernel(GemmArgs a) {
    constexpr int NWN = BN / WN;
    constexpr int NW = (BM / WM) * NWN;
    constexpr int NT = NW * 64;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int PITCH = BK + 8;            // bf16 elements per LDS row
    constexpr int CPR = BK / 8;              // 16-byte chunks per row
    constexpr int AC = BM * CPR / NT, BC = BN * CPR / NT;
    static_assert(AC * NT == BM * CPR && BC * NT == BN * CPR, "tile/thread mismatch");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2][(BM + BN) * PITCH];
    __shared__ double red[NW];

    if (a.state && a.state->halted) return;
    const SchedView sv = sched_view(a);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    const int64_t tiles_m = (a.I + BM - 1) / BM;
    const int L = remap_block();
    const int64_t tile_m = L % tiles_m, tile_n = L / tiles_m;
    const int64_t m0 = tile_m * BM, n0 = tile_n * BN;

    const uint16_t* Ab = static_cast<const uint16_t*>(a.A.base);
    const uint16_t* Bb = static_cast<const uint16_t*>(a.B.base);
    int64_t aoff[AC], boff[BC];
#pragma unroll
    for (int q = 0; q < AC; ++q) {
        const int c = tid + q * NT;
        const int64_t i = m0 + c / CPR;
        aoff[q] = (i < a.I) ? row_offset(a.A, sv, i) + (c % CPR) * 8 : -1;
    }
#pragma unroll
    for (int q = 0; q < BC; ++q) {
        const int c = tid + q * NT;
        const int64_t j = n0 + c / CPR;
        boff[q] = (j < a.J) ? row_offset(a.B, sv, j) + (c % CPR) * 8 : -1;
    }

    uint4 ra[AC], rb[BC];
    auto gload = [&](int64_t k0) {
        const int64_t ca = col_offset(a.A, sv, k0), cb = col_offset(a.B, sv, k0);
#pragma unroll
        for (int q = 0; q < AC; ++q) {
            const int kk = ((tid + q * NT) % CPR) * 8;
            ra[q] = (aoff[q] >= 0 && k0 + kk < a.R) ? *reinterpret_cast<const uint4*>(Ab + aoff[q] + ca)
                                                     : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < BC; ++q) {
            const int kk = ((tid + q * NT) % CPR) * 8;
            rb[q] = (boff[q] >= 0 && k0 + kk < a.R) ? *reinterpret_cast<const uint4*>(Bb + boff[q] + cb)
                                                     : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
        uint16_t* As = smem[buf];
        uint16_t* Bs = smem[buf] + BM * PITCH;
#pragma unroll
        for (int q = 0; q < AC; ++q) {
            const int c = tid + q * NT;
            *reinterpret_cast<uint4*>(As + (c / CPR) * PITCH + (c % CPR) * 8) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < BC; ++q) {
            const int c = tid + q * NT;
            *reinterpret_cast<uint4*>(Bs + (c / CPR) * PITCH + (c % CPR) * 8) = rb[q];
        }
    };

    floatx16 acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.0f;

    const int64_t nk = (a.R + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int frow = lane & 31, fk = (lane >> 5) * 8;
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const uint16_t* As = smem[buf] + (wm * WM + frow) * PITCH + fk;
        const uint16_t* Bs = smem[buf] + BM * PITCH + (wn * WN + frow) * PITCH + fk;
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) af[tm] = *reinterpret_cast<const bf16x8*>(As + tm * 32 * PITCH + ks);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) bfr[tn] = *reinterpret_cast<const bf16x8*>(Bs + tn * 32 * PITCH + ks);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm], bfr[tn], acc[tm][tn], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    epilogue<TM, TN, EPI>(a, sv, acc, m0 + wm * WM, n0 + wn * WN, lane, red);
    if (EPI == EPI_LOSS) {
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int w = 0; w < NW; ++w) s += red[w];
            a.partials[L] = s;
        }
    }
}

// ------------------------------------------------------------------ fp32 --
template <int BM, int BN, int BK, int WM, int WN, int EPI>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64) gemm_f32_kernel(GemmArgs a) {
    constexpr int NWN = BN / WN;
    constexpr int NW = (BM / WM) * NWN;
    constexpr int NT = NW * 64;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int PITCH = BK + 4;            // floats per LDS row
    constexpr int CPR = BK / 4;              // 16-byte chunks per row
    constexpr int AC = BM * CPR / NT, BC = BN * CPR / NT;
    static_assert(AC * NT == BM * CPR && BC * NT == BN * CPR, "tile/thread mismatch");
    __shared__ __attribute__((aligned(16))) float smem[2][(BM + BN) * PITCH];
    __shared__ double red[NW];

    if (a.state && a.state->halted) return;
    const SchedView sv = sched_view(a);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    const int64_t tiles_m = (a.I + BM - 1) / BM;
    const int L = remap_block();
    const int64_t tile_m = L % tiles_m, tile_n = L / tiles_m;
    const int64_t m0 = tile_m * BM, n0 = tile_n * BN;

    const float* Ab = static_cast<const float*>(a.A.base);
    const float* Bb = static_cast<const float*>(a.B.base);
    int64_t aoff[AC], boff[BC];
#pragma unroll
    for (int q = 0; q < AC; ++q) {
        const int c = tid + q * NT;
        const int64_t i = m0 + c / CPR;
        aoff[q] = (i < a.I) ? row_offset(a.A, sv, i) + (c % CPR) * 4 : -1;
    }
#pragma unroll
    for (int q = 0; q < BC; ++q) {
        const int c = tid + q * NT;
        const int64_t j = n0 + c / CPR;
        boff[q] = (j < a.J) ? row_offset(a.B, sv, j) + (c % CPR) * 4 : -1;
    }
    float4 ra[AC], rb[BC];
    auto gload = [&](int64_t k0) {
        const int64_t ca = col_offset(a.A, sv, k0), cb = col_offset(a.B, sv, k0);
#pragma unroll
        for (int q = 0; q < AC; ++q) {
            const int kk = ((tid + q * NT) % CPR) * 4;
            ra[q] = (aoff[q] >= 0 && k0 + kk < a.R) ? *reinterpret_cast<const float4*>(Ab + aoff[q] + ca)
                                                     : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int q = 0; q < BC; ++q) {
            const int kk = ((tid + q * NT) % CPR) * 4;
            rb[q] = (boff[q] >= 0 && k0 + kk < a.R) ? *reinterpret_cast<const float4*>(Bb + boff[q] + cb)
                                                     : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto sstore = [&](int buf) {
        float* As = smem[buf];
        float* Bs = smem[buf] + BM * PITCH;
#pragma unroll
        for (int q = 0; q < AC; ++q) {
            const int c = tid + q * NT;
            *reinterpret_cast<float4*>(As + (c / CPR) * PITCH + (c % CPR) * 4) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < BC; ++q) {
            const int c = tid + q * NT;
            *reinterpret_cast<float4*>(Bs + (c / CPR) * PITCH + (c % CPR) * 4) = rb[q];
        }
    };

    floatx16 acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.0f;

    const int64_t nk = (a.R + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int frow = lane & 31, fk = lane >> 5;
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const float* As = smem[buf] + (wm * WM + frow) * PITCH + fk;
        const float* Bs = smem[buf] + BM * PITCH + (wn * WN + frow) * PITCH + fk;
#pragma unroll
        for (int ks = 0; ks < BK; ks += 2) {
            float af[TM], bfr[TN];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) af[tm] = As[tm * 32 * PITCH + ks];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) bfr[tn] = Bs[tn * 32 * PITCH + ks];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[tm], bfr[tn], acc[tm][tn], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    epilogue<TM, TN, EPI>(a, sv, acc, m0 + wm * WM, n0 + wn * WN, lane, red);
    if (EPI == EPI_LOSS) {
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int w = 0; w < NW; ++w) s += red[w];
            a.partials[L] = s;
        }
    }
}

// Tile shapes.  bf16: 256 x 256 workgroup tiles of four 128 x 128 wavefront
// tiles (16 MFMA blocks each) when the problem yields at least one tile per
// CU, else 256 x 128 (four 128 x 64 wavefront tiles).  fp32: 128 x 128.
constexpr int kBK16 = 64;
constexpr int kBK32 = 32;

bool use_wide(int64_t I, int64_t J) {
    const int64_t wide = ((I + 255) / 256) * ((J + 255) / 256);
    return wide >= 256;
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_bf16_cfg(const GemmArgs& a, int32_t* nblocks, hipStream_t stream) {
    const int64_t tiles = ((a.I + BM - 1) / BM) * ((a.J + BN - 1) / BN);
    constexpr int NT = (BM / WM) * (BN / WN) * 64;
    if (a.epi == EPI_LOSS)
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, kBK16, WM, WN, EPI_LOSS>), dim3((unsigned)tiles), dim3(NT), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, kBK16, WM, WN, EPI_STORE>), dim3((unsigned)tiles), dim3(NT), 0,
                           stream, a);
    if (nblocks) *nblocks = (int32_t)tiles;
    return hipGetLastError();
}

}  // namespace

int32_t gemm_grid_blocks(bool bf16, int64_t I, int64_t J) {
    if (bf16) {
        if (use_wide(I, J)) return (int32_t)(((I + 255) / 256) * ((J + 255) / 256));
        return (int32_t)(((I + 255) / 256) * ((J + 127) / 128));
    }
    return (int32_t)(((I + 127) / 128) * ((J + 127) / 128));
}

hipError_t launch_gemm_bf16(const GemmArgs& a, int32_t* nblocks, hipStream_t stream) {
    if (use_wide(a.I, a.J)) return launch_bf16_cfg<256, 256, 128, 128>(a, nblocks, stream);
    return launch_bf16_cfg<256, 128, 128, 64>(a, nblocks, stream);
}

hipError_t launch_gemm_f32(const GemmArgs& a, int32_t* nblocks, hipStream_t stream) {
    const int64_t tiles = ((a.I + 127) / 128) * ((a.J + 127) / 128);
    if (a.epi == EPI_LOSS)
        hipLaunchKernelGGL((gemm_f32_kernel<128, 128, kBK32, 64, 64, EPI_LOSS>), dim3((unsigned)tiles), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<128, 128, kBK32, 64, 64, EPI_STORE>), dim3((unsigned)tiles), dim3(256), 0,
                           stream, a);
    if (nblocks) *nblocks = (int32_t)tiles;
    return hipGetLastError();
}

}  // namespace ar
