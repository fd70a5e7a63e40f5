// Device code of one block's stochastic interpolation and fixed-width
// packing for blocks of 4096 contiguous entries, shared by the quantizer
// (kvq_quant.hip) and the one-launch decode admission (kvq_eval16.hip).
//
// Page "Rate-adaptive KV-cache quantizer", Key formulas (3): an entry x in
// [q_i, q_{i+1}] becomes q_{i+1} with probability p = (x - q_i)/(q_{i+1} - q_i)
// and q_i otherwise; Implementation notes: the codebook, the symbol stream
// and the block lengths are stored.
//
// Lane t of a kThreads-thread workgroup owns the 8-entry chunks t, t +
// kThreads, ...  A chunk's eight w-bit codes are exactly w bytes of the
// block's little-endian stream (chunk c at byte w c), so loads are 16-byte
// coalesced and stores need no cross-lane packing.  The draw of entry t of
// block r is word t & 3 of Philox4x32-10 on counter (t >> 2, r lo, r hi, 0)
// under key (seed lo, seed hi).
#pragma once

#include "kvq_internal.h"

namespace kvq {

// An 8-entry chunk as loaded (fp16: 16 bytes in w[0]; fp32: 32 bytes), kept
// apart from its conversion so that the next chunk's load can be issued
// before this chunk is used.
template <int kDt>
__device__ __forceinline__ void load_raw8(const void* src, int64_t e0, uint4 (&w)[2]) {
    if (kDt == KVQ_F16) {
        w[0] = *reinterpret_cast<const uint4*>(reinterpret_cast<const __half*>(src) + e0);
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(src) + e0);
        w[0] = p[0];
        w[1] = p[1];
    }
}

template <int kDt>
__device__ __forceinline__ void unpack8(const uint4 (&w)[2], float* x) {
    if (kDt == KVQ_F16) {
        const uint32_t h[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = __half2float(__ushort_as_half((unsigned short)(h[k] & 0xffffu)));
            x[2 * k + 1] = __half2float(__ushort_as_half((unsigned short)(h[k] >> 16)));
        }
    } else {
        const uint32_t f[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = __uint_as_float(f[k]);
    }
}

__device__ __forceinline__ void store_bytes(uint8_t* dst, uint32_t bits, int w) {
    switch (w) {
    case 1: dst[0] = (uint8_t)bits; break;
    case 2: *reinterpret_cast<uint16_t*>(dst) = (uint16_t)bits; break;
    case 3:
        if (((uintptr_t)dst & 1u) == 0) {
            *reinterpret_cast<uint16_t*>(dst) = (uint16_t)bits;
            dst[2] = (uint8_t)(bits >> 16);
        } else {
            dst[0] = (uint8_t)bits;
            *reinterpret_cast<uint16_t*>(dst + 1) = (uint16_t)(bits >> 8);
        }
        break;
    default: *reinterpret_cast<uint32_t*>(dst) = bits; break;
    }
}

// Interval lookup of quantize4096.  Entry x maps to the value-space cell
// c = RN(x sc + A) - 1.5 2^23 (one fma: in [2^23, 2^24) an fp32 is an
// integer, so the sum's bits are the cell), with sc = (kQCells - 1) / (q_max
// - q_min) and A = RN(1.5 2^23 - q_min sc).  Both roundings together move c
// by less than one cell from (x - q_min) sc, so every x of cell c lies in
// u-space [c - 1.0625, c + 1.0625].  The cell's record holds the interval
// index i_lo of the lower end of that range and t = q_{i_lo + 1}: unless a
// second codepoint lies inside the range (the cell is then flagged and its
// entries take a binary search), x lies in interval i_lo + (x >= t).
constexpr int kQCells = 512;
constexpr int kQLut = kQCells + 2;            // cells -1 .. kQCells
constexpr int kQLutPer = (kQLut + 63) / 64;   // cells per lane of the build (one wave)
constexpr uint32_t kCellSlow = 0x80000000u;   // record flag: two or more codepoints in range
constexpr float kMagic = 12582912.0f;         // 1.5 2^23
constexpr uint32_t kMagicBits = 0x4B400000u;

// Largest interval index i with q[i] <= x over 16 slots padded with +inf
// (i = m - 1 only for x equal to the maximum).
__device__ __forceinline__ uint32_t search16(const float* q, float x) {
    const char* qb = reinterpret_cast<const char*>(q);
    uint32_t o = 0;
    o = (*reinterpret_cast<const float*>(qb + o + 32) <= x) ? o + 32 : o;
    o = (*reinterpret_cast<const float*>(qb + o + 16) <= x) ? o + 16 : o;
    o = (*reinterpret_cast<const float*>(qb + o + 8) <= x) ? o + 8 : o;
    o = (*reinterpret_cast<const float*>(qb + o + 4) <= x) ? o + 4 : o;
    return o >> 2;
}

// LDS of one block's quantization.
struct QuantLds {
    float qs[kMaxS + 1];            // codepoints, +inf from slot m on
    float2 rec[kMaxS + 1];          // (q_i, 2^24 / (q_{i+1} - q_i)); 0 from slot m - 1 on
    union {
        uint2 lut[kQLut];             // cell c + 1: (i_lo | kCellSlow, bits of t)
        uint32_t diff[kQLutPer * 64]; // build: difference counts per cell (read by
                                      // the one building wave before it writes lut)
    };
};
static_assert(kQLutPer * 64 * 4 <= kQLut * 8, "the build counts fit the table");

// Quantize and pack block r (4096 contiguous entries) whose codebook value
// for this lane (slot tid, +inf past s), level count and word offset have
// been loaded, as has its data: chunk h of this lane (entries 8 (tid + h
// kThreads) .. + 7) in chunks[h] for fp16, or loaded here one step ahead for
// fp32 (src, e_base).
// kDefer: the codes are not stored; chunk h's bits go to bits_out[h] (the
// caller stores them once the block's word offset is known) and the code
// width is returned (0: nothing to store).
template <int kThreads, int kDt, bool kDefer = false>
__device__ __forceinline__ int quantize_block4096(QuantLds& L, int64_t r, int s, float cbv, int mraw,
                                                  uint64_t ob, const uint4 (&chunks)[512 / kThreads][2],
                                                  const void* src, int64_t e_base, uint32_t k0, uint32_t k1,
                                                  uint32_t* __restrict__ codes,
                                                  uint32_t* bits_out = nullptr) {
    const int tid = threadIdx.x;
    constexpr int kNH = 512 / kThreads;
    constexpr bool kAllAhead = kDt == KVQ_F16;
    uint4 cur[2] = {}, nxt[2] = {};
    if (!kAllAhead) load_raw8<kDt>(src, e_base + 8 * tid, cur);
    const int m = min(max(mraw, 1), s);
    const int w = code_width(m);
    if (tid <= kMaxS) L.qs[tid] = tid < m ? cbv : __builtin_huge_valf();
    for (int i = tid; i < kQLutPer * 64; i += kThreads) L.diff[i] = 0u;
    __syncthreads();
    if (w == 0) return 0;  // one level: no code bits (uniform over the block)
    // per-interval records; an interval whose inverse width is not finite
    // (fp32 codepoints closer than ~2^-102 of each other) sends the block to
    // the exact division below
    bool bad_inv = false;
    if (tid <= kMaxS) {
        const float a = L.qs[tid];
        float iv = 0.0f;
        if (tid < m - 1) {
            iv = 0x1p24f / (L.qs[tid + 1] - a);
            bad_inv = !(iv < __builtin_huge_valf());
        }
        L.rec[tid] = make_float2(a, iv);
    }
    // cell geometry (uniform): usable when q_min sc and q_max sc stay within
    // 2^21, so that A and every x sc + A are exact-integer-range floats
    const float mn = L.qs[0], mx = L.qs[m - 1];
    const float sc = (float)((double)(kQCells - 1) / ((double)mx - (double)mn));
    const double dsc = (double)sc;
    const bool cells_ok = sc < __builtin_huge_valf() && fabs((double)mn * dsc) <= 0x1p21 &&
                          fabs((double)mx * dsc) <= 0x1p21;
    const float A = (float)((double)kMagic - (double)mn * dsc);
    if (cells_ok && tid >= 1 && tid < m) {
        // codepoint tid at u = (q - q_min) sc: below the whole range of
        // cells c >= ceil(u + 1.0625) (counts toward their i_lo), inside or
        // below that of cells c >= ceil(u - 1.0625) (toward their upper count)
        const double u = ((double)L.qs[tid] - (double)mn) * dsc;
        const double clo = ceil(u + 1.0625), chi = ceil(u - 1.0625);
        if (clo <= (double)kQCells) atomicAdd(&L.diff[(int)clo + 1], 1u);
        if (chi <= (double)kQCells) atomicAdd(&L.diff[chi < -1.0 ? 0 : (int)chi + 1], 1u << 16);
    }
    const int slow_div = __syncthreads_or(bad_inv ? 1 : 0);
    if (cells_ok) {
        // inclusive prefix of the counts over cells (one wave: lane l owns
        // cells l kQLutPer .. l kQLutPer + kQLutPer - 1)
        if (tid < 64) {
            uint32_t v[kQLutPer];
            uint32_t run = 0;
#pragma unroll
            for (int k = 0; k < kQLutPer; ++k) {
                run += L.diff[tid * kQLutPer + k];
                v[k] = run;
            }
            const uint32_t incl = wave_scan_add_u32(run);
            const uint32_t base = incl - run;
#pragma unroll
            for (int k = 0; k < kQLutPer; ++k) {
                const int cell = tid * kQLutPer + k;
                if (cell < kQLut) {
                    const uint32_t cnt = base + v[k];
                    const uint32_t ilo = cnt & 0xffffu, hi = cnt >> 16;
                    L.lut[cell] = make_uint2(ilo | (hi >= ilo + 2u ? kCellSlow : 0u), __float_as_uint(L.qs[ilo + 1]));
                }
            }
        }
    }
    __syncthreads();
    uint8_t* out = kDefer ? nullptr : reinterpret_cast<uint8_t*>(codes + ob);
    const uint32_t rlo = (uint32_t)r, rhi = (uint32_t)((uint64_t)r >> 32);
    // byte offset of lut[c + 1] from the bits of x sc + A
    constexpr uint32_t kLutOff = 8u - (kMagicBits << 3);
    constexpr uint32_t kLutLast = 8u * (kQLut - 1);
    const char* lutb = reinterpret_cast<const char*>(L.lut);
    const char* recb = reinterpret_cast<const char*>(L.rec);
    const bool fast = cells_ok && !slow_div;
#pragma unroll
    for (int half = 0; half < kNH; ++half) {
        const int ch = tid + half * kThreads;
        float x[8];
        if (kAllAhead) {
            unpack8<kDt>(chunks[half], x);
        } else {
            if (half + 1 < kNH) load_raw8<kDt>(src, e_base + 8 * (ch + kThreads), nxt);
            unpack8<kDt>(cur, x);
        }
        uint32_t wd[8];
        {
            uint32_t a0 = (uint32_t)(2 * ch), a1 = rlo, a2 = rhi, a3 = 0u;
            philox4x32_10(a0, a1, a2, a3, k0, k1);
            uint32_t b0 = (uint32_t)(2 * ch + 1), b1 = rlo, b2 = rhi, b3 = 0u;
            philox4x32_10(b0, b1, b2, b3, k0, k1);
            wd[0] = a0; wd[1] = a1; wd[2] = a2; wd[3] = a3;
            wd[4] = b0; wd[5] = b1; wd[6] = b2; wd[7] = b3;
        }
        uint32_t code[8];
        uint32_t flags = 0;
        if (fast) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xv = x[e];
                const float y = fmaf(xv, sc, A);
                // clamp: a non-finite x cannot leave the table
                const uint32_t ca = min((__float_as_uint(y) << 3) + kLutOff, kLutLast);
                const uint2 cl = *reinterpret_cast<const uint2*>(__builtin_assume_aligned(lutb + ca, 8));
                const uint32_t i = cl.x + (xv >= __uint_as_float(cl.y) ? 1u : 0u);
                // the flag bit of i is shifted out of the record offset
                const float2 qi = *reinterpret_cast<const float2*>(__builtin_assume_aligned(recb + (i << 3), 8));
                // p 2^24 against the 24-bit draw (word >> 8): u < p without
                // scaling u; p outside [0, 1] by round-off decides the same
                // way as its clamp
                const float p24 = (xv - qi.x) * qi.y;
                const float u24 = (float)(wd[e] >> 8);
                // code = i + (u24 < p24): one compare and the carry added to
                // i (written out, since the compiler otherwise rebuilds i
                // here from a 0/1 copy of the earlier comparison, one more
                // instruction per entry: 1.58 -> 1.49 ms on the long-context
                // cache without it)
                asm("v_cmp_lt_f32_e32 vcc, %1, %2\n\ts_nop 1\n\tv_addc_co_u32_e32 %0, vcc, 0, %3, vcc"
                    : "=v"(code[e]) : "v"(u24), "v"(p24), "v"(i) : "vcc");
                flags |= cl.x;
            }
        }
        if (!fast || (flags & kCellSlow)) {
            // flagged cells (or a block without usable cells): binary search,
            // and the exact division where an inverse width overflowed
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xv = x[e];
                if (!fast || (code[e] & kCellSlow)) {
                    const uint32_t i = search16(L.qs, xv);
                    const float2 qi = L.rec[i];
                    bool up;
                    if (slow_div) {
                        const float b = L.qs[min(i + 1u, (uint32_t)kMaxS)];
                        const float p = (xv - qi.x) / (b - qi.x);  // +inf width at the maximum: p = 0
                        up = (float)(wd[e] >> 8) * 0x1p-24f < p;
                    } else {
                        up = (float)(wd[e] >> 8) < (xv - qi.x) * qi.y;
                    }
                    code[e] = i + (up ? 1u : 0u);
                }
            }
        }
        uint32_t bits = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) bits |= code[e] << (w * e);
        if (kDefer)
            bits_out[half] = bits;
        else
            store_bytes(out + w * ch, bits, w);
        cur[0] = nxt[0];
        cur[1] = nxt[1];
    }
    return w;
}

}  // namespace kvq
