// INT4-weight x bf16-activation GEMM on the packed output of the quantizer:
// Y[m, n] = sum_k X[m, k] * bf16(s[n, k/g] * (q[n, k] - z[n, k/g])).
//
// This is the deployment form of the tuned layer: the AutoRound blog (sec. 4,
// the QDQ-versus-real-INT4 comparison) contrasts the fake-quantized FP GEMM
// used while tuning with a kernel that reads 4-bit codes and dequantizes them
// inside the GEMM, and the coordinates page (sec. 2-3) lists the packed
// weight, per-group scale and zero-point as what such a kernel consumes.  The
// dequantized operand is the same bf16 rounding of the fp32 s * (q - z) that
// the quantizer produces, so the GEMM equals X times the bf16 fake-quantized
// weight.
//
// Mapping (C[i, j] = sum_r A[i, r] * B[j, r] as in the tuning GEMMs):
//   A = X [M, K] bf16 and B = the weight, read as packed codes (one dword =
//   8 codes along k) with their group's scale and zero.  Both are loaded into
//   registers two k-steps ahead of use; per k-step of 64 every thread writes
//   its X chunks and its dequantized weight chunks (each weight dequantized
//   once per tile) into one of two LDS stages.  Register staging rather than
//   LDS DMA: the codes must pass through registers to be dequantized, and
//   the compiler cannot order DMA completions against register loads on the
//   one vmcnt counter, so mixing the two drains the DMA queue every step.
// LDS rows are 128 bytes with the XOR swizzle of the tuning GEMMs, so the
// 16-byte writes and the fragment reads are bank-conflict free.
// Accumulation is fp32 in v_mfma_f32_32x32x16_bf16.
#include <type_traits>

#include "ar_internal.h"
#include "gemm_tiles.h"
#include "w4a16.h"

namespace ar {
namespace {

using gemm::bf16x8;
using gemm::floatx16;
using gemm::gbl_void;
using gemm::lds_void;
// native 16-byte vector: HIP's uint4 wraps a union, which keeps arrays of it
// out of registers
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup barrier after this wave's LDS writes have completed.  Unlike
// __syncthreads() it does not wait for outstanding global loads, which are
// the prefetches of later k-steps.
__device__ __forceinline__ void lds_write_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Eight consecutive codes (one packed dword, low nibble first) -> eight bf16
// weights.  v_perm_b32 places a nibble byte under the exponent byte 0x4B, so
// the float is 2^23 + q exactly; subtracting 2^23 + z leaves q - z exactly,
// and one fp32 multiply by s gives the quantizer's s * (q - z).  The bf16
// conversion rounds to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ u32x4 dequant8(uint32_t p, float s, float zf) {
    const uint32_t lo = p & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6
    const uint32_t hi = (p >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
    const uint32_t magic = 0x4B000000u;
    const float off = 8388608.0f + zf;
    float w[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        // result bytes: [byte b of lo|hi, 0, 0, 0x4B]
        const uint32_t sel = 0x070C0C00u | (uint32_t)b;
        w[2 * b] = s * (__uint_as_float(__builtin_amdgcn_perm(magic, lo, sel)) - off);
        w[2 * b + 1] = s * (__uint_as_float(__builtin_amdgcn_perm(magic, hi, sel)) - off);
    }
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16x2 v;
        v[0] = (__bf16)w[2 * e];
        v[1] = (__bf16)w[2 * e + 1];
        o[e] = __builtin_bit_cast(uint32_t, v);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

template <int BM, int BN, int NWM, int NWN, bool OUT_BF16>
__global__ void __launch_bounds__(NWM * NWN * 64) w4a16_gemm_kernel(W4A16Args a) {
    constexpr int BK = 64;
    constexpr int NW = NWM * NWN;
    constexpr int NT = NW * 64;
    constexpr int WM = BM / NWM, WN = BN / NWN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int ROWB = BK * 2;          // bytes per LDS row
    constexpr int SLOTS = BK / 8;         // 16-byte chunks per row
    constexpr int RPW = 256 / ROWB;       // rows per 256-byte bank window
    constexpr int A_STAGE = BM * ROWB;
    constexpr int B_STAGE = BN * ROWB;
    constexpr int ACT = BM * SLOTS / NT;  // X chunks per thread per k-step
    constexpr int CPT = BN * SLOTS / NT;  // weight chunks per thread per k-step
    static_assert(ACT * NT == BM * SLOTS && CPT * NT == BN * SLOTS, "chunks must split evenly over threads");
    static_assert(TM >= 1 && TN >= 1, "wavefront tile below one MFMA block");
    __shared__ __attribute__((aligned(1024))) char sa0[A_STAGE];
    __shared__ __attribute__((aligned(1024))) char sa1[A_STAGE];
    __shared__ __attribute__((aligned(1024))) char sb0[B_STAGE];
    __shared__ __attribute__((aligned(1024))) char sb1[B_STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
    int64_t tile_m, tile_n;
    gemm::tile_coords<BM, BN>(tiles_m, tiles_n, tile_m, tile_n);
    const int64_t m0 = tile_m * BM, n0 = tile_n * BN;
    const int nk = (int)(a.K / BK);

    // Chunk c = tid + q NT of a tile is row c / SLOTS, 8 elements starting at
    // 8 (c % SLOTS) of the k-step; every chunk of a thread has the same
    // c % SLOTS.  Rows past M or N are clamped (their results are not stored).
    const int c8 = tid % SLOTS;
    int64_t xrow[ACT];
    int aoff[ACT];
#pragma unroll
    for (int q = 0; q < ACT; ++q) {
        const int row = (tid + q * NT) / SLOTS;
        int64_t m = m0 + row;
        if (m >= a.M) m = a.M - 1;
        xrow[q] = m * a.ldx + c8 * 8;
        aoff[q] = row * ROWB + ((c8 ^ ((row / RPW) % SLOTS)) << 4);
    }
    int64_t prow[CPT], grow[CPT];
    int boff[CPT];
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
        const int row = (tid + q * NT) / SLOTS;
        int64_t n = n0 + row;
        if (n >= a.N) n = a.N - 1;
        prow[q] = n * (a.K / 8) + c8;
        grow[q] = n * a.G;
        boff[q] = row * ROWB + ((c8 ^ ((row / RPW) % SLOTS)) << 4);
    }

    // Two register sets, one per parity of the k-step, as separate arrays
    // selected at compile time: with a runtime-indexed 2-D array the compiler
    // moves the set into LDS or scratch instead of registers.
    struct RegSet {
        u32x4 x[ACT];
        uint32_t pk[CPT];
        float sc[CPT];
        uint32_t zr[CPT];
    };
    RegSet r0, r1;
    auto load = [&](RegSet& r, int kt) __attribute__((always_inline)) {
        // steps past the end reload the last one (never used), so no branch
        const int kk = kt < nk ? kt : nk - 1;
        const int grp = (kk * BK + c8 * 8) / a.g;
#pragma unroll
        for (int q = 0; q < ACT; ++q) r.x[q] = *reinterpret_cast<const u32x4*>(a.X + xrow[q] + (int64_t)kk * BK);
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            r.pk[q] = a.packed[prow[q] + (int64_t)kk * SLOTS];
            r.sc[q] = a.scale[grow[q] + grp];
            r.zr[q] = a.zero[grow[q] + grp];
        }
    };
    auto store = [&](const RegSet& r, char* as, char* bs) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < ACT; ++q) *reinterpret_cast<u32x4*>(as + aoff[q]) = r.x[q];
#pragma unroll
        for (int q = 0; q < CPT; ++q)
            *reinterpret_cast<u32x4*>(bs + boff[q]) = dequant8(r.pk[q], r.sc[q], (float)r.zr[q]);
    };

    floatx16 acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.0f;

    // Step 0 goes to LDS stage 0; steps 1 and 2 are in flight in registers.
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    load(r0, 0);
    load(r1, 1);
    store(r0, sa0, sb0);
    load(r0, 2);

    const int frow = lane & 31, fhalf = lane >> 5;
    auto frag = [&](const char* base, int row, int c) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(base + row * ROWB + ((c ^ ((row / RPW) % SLOTS)) << 4));
    };
    // k-step kt of parity P: MFMAs on LDS stage P; halfway, the registers of
    // step kt + 1 go to LDS stage P ^ 1 (read by all waves in step kt - 1,
    // which every wave finished before this step's barrier) and are refilled
    // with step kt + 3.
    auto step = [&](int kt, auto par) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        lds_write_barrier();
        const char* As = P == 0 ? sa0 : sa1;
        const char* Bs = P == 0 ? sb0 : sb1;
        constexpr int KS = BK / 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) af[tm] = frag(As, wm * WM + tm * 32 + frow, ks * 2 + fhalf);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) bfr[tn] = frag(Bs, wn * WN + tn * 32 + frow, ks * 2 + fhalf);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm], bfr[tn], acc[tm][tn], 0, 0, 0);
            // unconditional, so every step issues the same loads and the
            // compiler's wait counts stay exact: past the end the loads are
            // clamped repeats and the LDS stage written is read by no one
            if (ks == KS / 2 - 1) {
                RegSet& r = P == 0 ? r1 : r0;
                store(r, P == 0 ? sa1 : sa0, P == 0 ? sb1 : sb0);
                load(r, kt + 3);
            }
        }
    };
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
        step(kt, I0{});
        step(kt + 1, I1{});
    }
    if (kt < nk) step(kt, I0{});
    gemm::wait_vmcnt<0>();   // the last, unused prefetches

    const int half = lane >> 5, cl = lane & 31;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int64_t n = n0 + wn * WN + tn * 32 + cl;
        if (n >= a.N) continue;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * WM + tm * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                if (m >= a.M) continue;
                if constexpr (OUT_BF16)
                    static_cast<uint16_t*>(a.Y)[m * a.ldy + n] = f32_to_bf16(acc[tm][tn][r]);
                else
                    static_cast<float*>(a.Y)[m * a.ldy + n] = acc[tm][tn][r];
            }
        }
    }
}

// Small batches (17 to 64 rows; up to 16 go to the decode kernel below):
// streaming the packed weight once is the bound, so there is no LDS staging.  A workgroup of 16 wavefronts owns 16
// weight rows; its wavefronts take turns over K in super-steps of 128 (wave
// w handles super-steps w, w + 16, ...), so each row's codes are read once,
// and the partial sums meet in LDS at the end (fixed order, deterministic).
// v_mfma_f32_16x16x32_bf16: lane l supplies row l % 16 of the 16 x 32 A and
// B tiles and k-chunk l / 16.  Within a super-step the k order is permuted
// identically for both operands (lane group c, MFMA j -> k = 128 s + 32 c +
// 8 j), so a lane's codes for the four MFMAs are 16 contiguous bytes.  Each
// dequantized chunk feeds MB MFMAs, one per 16-row block of X.
template <int MB, bool OUT_BF16, bool G128>
__global__ void __launch_bounds__(1024) w4a16_skinny_kernel(W4A16Args a) {
    constexpr int NWAVE = 16;
    typedef float floatx4 __attribute__((ext_vector_type(4)));
    __shared__ float red[NWAVE][MB][16][16];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, c = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    int64_t n = n0 + r16;
    if (n >= a.N) n = a.N - 1;
    const uint8_t* prow = reinterpret_cast<const uint8_t*>(a.packed) + n * (a.K / 2);
    const float* srow = a.scale + n * a.G;
    const uint8_t* zrow = a.zero + n * a.G;
    const uint16_t* xrow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        int64_t m = mb * 16 + r16;
        if (m >= a.M) m = a.M - 1;
        xrow[mb] = a.X + m * a.ldx;
    }
    floatx4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // Two register sets, one super-step in flight while the other computes;
    // every iteration issues the same loads (clamped past the end) so the
    // compiler's wait counts stay exact.
    struct Regs {
        u32x4 codes;
        float sj[4];
        uint32_t zj[4];
        u32x4 x[MB][4];
    };
    const int nss = (int)(a.K / 128);
    auto load = [&](Regs& R, int ss) __attribute__((always_inline)) {
        if (ss >= nss) ss = nss - 1;
        const int kb = ss * 128 + c * 32;
        R.codes = *reinterpret_cast<const u32x4*>(prow + kb / 2);
        if constexpr (G128) {
            // a 128-aligned super-step lies in one group
            const int grp = (ss * 128) / a.g;
            R.sj[0] = srow[grp];
            R.zj[0] = zrow[grp];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int grp = (kb + 8 * j) / a.g;
                R.sj[j] = srow[grp];
                R.zj[j] = zrow[grp];
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j) R.x[mb][j] = *reinterpret_cast<const u32x4*>(xrow[mb] + kb + 8 * j);
    };
    auto compute = [&](const Regs& R) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int jj = G128 ? 0 : j;
            const bf16x8 wf = __builtin_bit_cast(bf16x8, dequant8(R.codes[j], R.sj[jj], (float)R.zj[jj]));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, R.x[mb][j]), wf,
                                                                  acc[mb], 0, 0, 0);
        }
    };
    const int niter = wave < nss ? (nss - wave + NWAVE - 1) / NWAVE : 0;
    if (niter > 0) {
        Regs R0, R1;
        load(R0, wave);
        int i = 0;
        for (; i + 2 <= niter; i += 2) {
            load(R1, wave + (i + 1) * NWAVE);
            compute(R0);
            load(R0, wave + (i + 2) * NWAVE);
            compute(R1);
        }
        if (i < niter) compute(R0);
    }

    // C of a 16 x 16 MFMA: lane l, element r -> row 4 (l / 16) + r, column l % 16
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][mb][4 * c + r][r16] = acc[mb][r];
    __syncthreads();
    for (int t = threadIdx.x; t < MB * 256; t += 1024) {
        const int mb = t / 256, i = (t / 16) % 16, j = t % 16;
        const int64_t m = mb * 16 + i, nn = n0 + j;
        if (m >= a.M || nn >= a.N) continue;
        float sum = 0.0f;
        for (int w = 0; w < NWAVE; ++w) sum += red[w][mb][i][j];
        if constexpr (OUT_BF16)
            static_cast<uint16_t*>(a.Y)[m * a.ldy + nn] = f32_to_bf16(sum);
        else
            static_cast<float*>(a.Y)[m * a.ldy + nn] = sum;
    }
}

// Decode batches of at most 16 tokens, K a multiple of 128, any K: no LDS
// staging.  Each 16-row MFMA tile uses every X fragment once, so X goes
// straight from the caches into registers; NW wavefronts own 16 weight rows
// and take the super-steps of 128 k in turn (wave w: w, w + NW, ...).  A
// round issues the codes, scales, zero-points and X fragments of NPW
// super-steps at once; the compiler's in-order waits then let the first
// super-step's dequantization and MFMAs run while later loads are in flight.
// Partial sums meet in LDS in wave order.  One or two tiles per workgroup
// launch with 16 wavefronts and two super-steps per round (a K of 4096 is
// one round): four times the wavefronts of a 4-wavefront form, whose
// dependent chain of loads, dequantization and MFMAs per wavefront was four
// times longer.
// GC: how a lane's 32 k of a super-step meet the groups.  0: the group
// size is a multiple of 128 (one scale per super-step); 1: a multiple of 32
// (one per lane); 2: smaller (one per 8 k).
template <bool OUT_BF16, int GC, int NW, int NPW, int RT>
__global__ void __launch_bounds__(64 * NW) w4a16_decode_kernel(W4A16Args a) {
    typedef float floatx4 __attribute__((ext_vector_type(4)));
    constexpr int NS = GC == 2 ? 4 : 1;   // scales per lane and super-step
    __shared__ float red[NW][RT][16][16];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, c = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * RT;
    const int nss = (int)(a.K / 128);
    const int64_t xr = r16 < a.M ? r16 : a.M - 1;   // rows at or past M: not stored
    const uint16_t* xrow = a.X + xr * a.ldx;
    const uint8_t* prow[RT];
    const float* srow[RT];
    const uint8_t* zrow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        int64_t n = n0 + rt * 16 + r16;
        if (n >= a.N) n = a.N - 1;
        prow[rt] = reinterpret_cast<const uint8_t*>(a.packed) + n * (a.K / 2);
        srow[rt] = a.scale + n * a.G;
        zrow[rt] = a.zero + n * a.G;
    }

    floatx4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int base = 0; base < nss; base += NW * NPW) {
        u32x4 codes[RT][NPW];
        bf16x8 xf[NPW][4];
        float sc[RT][NPW][NS];
        uint32_t zp[RT][NPW][NS];
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            int ss = base + wave + NW * i;
            if (ss >= nss) ss = nss - 1;
            const int kb = ss * 128 + c * 32;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) codes[rt][i] = *reinterpret_cast<const u32x4*>(prow[rt] + kb / 2);
#pragma unroll
            for (int j = 0; j < 4; ++j) xf[i][j] = *reinterpret_cast<const bf16x8*>(xrow + kb + 8 * j);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    const int gi = GC == 0 ? (ss * 128) / a.g : GC == 1 ? kb / a.g : (kb + 8 * j) / a.g;
                    sc[rt][i][j] = srow[rt][gi];
                    zp[rt][i][j] = zrow[rt][gi];
                }
        }
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
            if (base + wave + NW * i < nss) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int jj = NS == 1 ? 0 : j;
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const bf16x8 wf =
                            __builtin_bit_cast(bf16x8, dequant8(codes[rt][i][j], sc[rt][i][jj], (float)zp[rt][i][jj]));
                        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf[i][j], wf, acc[rt], 0, 0, 0);
                    }
                }
            }
        }
    }
    // C of a 16 x 16 MFMA: lane l, element r -> row 4 (l / 16) + r, column l % 16
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][rt][4 * c + r][r16] = acc[rt][r];
    __syncthreads();
    for (int t = threadIdx.x; t < 256 * RT; t += 64 * NW) {
        const int rt = t / 256, i = (t / 16) % 16, j = t % 16;
        const int64_t nn = n0 + rt * 16 + j;
        if (i < a.M && nn < a.N) {
            float sum = red[0][rt][i][j];
#pragma unroll
            for (int w = 1; w < NW; ++w) sum += red[w][rt][i][j];
            if constexpr (OUT_BF16)
                static_cast<uint16_t*>(a.Y)[i * a.ldy + nn] = f32_to_bf16(sum);
            else
                static_cast<float*>(a.Y)[i * a.ldy + nn] = sum;
        }
    }
}

template <int NW, int NPW, int RT>
void launch_decode_rt(const W4A16Args& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.N + 16 * RT - 1) / (16 * RT))), block(64 * NW);
    const int gc = a.g % 128 == 0 ? 0 : a.g % 32 == 0 ? 1 : 2;
    if (a.y_bf16) {
        if (gc == 0) hipLaunchKernelGGL((w4a16_decode_kernel<true, 0, NW, NPW, RT>), grid, block, 0, stream, a);
        else if (gc == 1) hipLaunchKernelGGL((w4a16_decode_kernel<true, 1, NW, NPW, RT>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((w4a16_decode_kernel<true, 2, NW, NPW, RT>), grid, block, 0, stream, a);
    } else {
        if (gc == 0) hipLaunchKernelGGL((w4a16_decode_kernel<false, 0, NW, NPW, RT>), grid, block, 0, stream, a);
        else if (gc == 1) hipLaunchKernelGGL((w4a16_decode_kernel<false, 1, NW, NPW, RT>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((w4a16_decode_kernel<false, 2, NW, NPW, RT>), grid, block, 0, stream, a);
    }
}

// RT 16-row tiles per workgroup share each X fragment: with one tile per
// workgroup every workgroup reads all of X (M rows of K), which for a long
// weight (N = 28672) moves 3.5x the packed weight's bytes through the L2s.
// More tiles per workgroup only while the grid still has 256 workgroups.
// Four tiles take 8 wavefronts with one super-step per round: 95 registers,
// so two workgroups share a CU and a 28672-row weight's 448 workgroups run
// in one round (two super-steps per round need 143 registers, one
// workgroup per CU and two rounds: 71 against 63 us).
void launch_decode_direct(const W4A16Args& a, hipStream_t stream) {
    if (a.N >= 16 * 4 * 256) launch_decode_rt<8, 1, 4>(a, stream);
    else if (a.N >= 16 * 2 * 256) launch_decode_rt<16, 2, 2>(a, stream);
    else launch_decode_rt<16, 2, 1>(a, stream);
}

template <int MB>
void launch_skinny(const W4A16Args& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.N + 15) / 16)), block(1024);
    const bool g128 = a.g % 128 == 0;
    if (a.y_bf16) {
        if (g128) hipLaunchKernelGGL((w4a16_skinny_kernel<MB, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((w4a16_skinny_kernel<MB, true, false>), grid, block, 0, stream, a);
    } else {
        if (g128) hipLaunchKernelGGL((w4a16_skinny_kernel<MB, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((w4a16_skinny_kernel<MB, false, false>), grid, block, 0, stream, a);
    }
}

}  // namespace

hipError_t launch_w4a16_gemm(const W4A16Args& a, hipStream_t stream) {
    if (a.M <= 16 && a.K % 128 == 0 && a.ldx % 8 == 0 && reinterpret_cast<uintptr_t>(a.X) % 16 == 0 &&
        reinterpret_cast<uintptr_t>(a.packed) % 16 == 0) {
        launch_decode_direct(a, stream);
        return hipGetLastError();
    }
    // (batches of at most 16 rows with these alignments took the decode kernel above)
    if (a.M > 16 && a.M <= 64 && a.K % 128 == 0 && reinterpret_cast<uintptr_t>(a.packed) % 16 == 0) {
        if (a.M <= 32) launch_skinny<2>(a, stream);
        else launch_skinny<4>(a, stream);
        return hipGetLastError();
    }
    constexpr int BM = 256, BN = 128, NWM = 4, NWN = 2;
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (a.y_bf16)
        hipLaunchKernelGGL((w4a16_gemm_kernel<BM, BN, NWM, NWN, true>), dim3((unsigned)tiles),
                           dim3(NWM * NWN * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((w4a16_gemm_kernel<BM, BN, NWM, NWN, false>), dim3((unsigned)tiles),
                           dim3(NWM * NWN * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace ar
