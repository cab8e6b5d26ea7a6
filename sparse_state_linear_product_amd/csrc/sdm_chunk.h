// Shared pieces of the chunk-parallel SDM recurrence (sdm_chunk.hip: forward,
// sdm_chunk_bwd.hip: backward): the chunk geometry and plan layout.  The LDS /
// LDS-DMA helpers the apply kernels use come from lds_dma.h.
#pragma once
#include <type_traits>
#include <utility>

#include "common.h"
#include "lds_dma.h"

namespace sslp {
namespace chunk {

constexpr int CW = 8;                // columns per apply workgroup (one 32-byte row piece)
constexpr int NWAVE = 8;             // wavefronts per apply workgroup
constexpr int NE = 512;              // write entries per chunk (C x W)
constexpr int JW = 32 / NWAVE;       // row DMAs per wavefront and chunk (32 per chunk)

// plan block of one (b, h, chunk), 32-bit words: a fixed part (layout below),
// then a tail of exception records, extra pairs and forward rows.  The fixed
// part and the first PL_TAILWIN words of the tail are staged in LDS; tail words
// past that (only with heavy slot reuse) are read from memory.
constexpr int PL_TAIL = 4096;
constexpr int PL_TAILWIN = 2048;
constexpr int PL_DMA_WORDS = PL_TAIL + PL_TAILWIN;  // 24 KB staged per chunk
constexpr int PL_WORDS = PL_TAIL + 2 * NE + 3 * NE + 2 * NE;  // worst-case tail
static_assert((PL_DMA_WORDS * 4) % 1024 == 0 && (PL_WORDS * 4) % 16 == 0, "plan DMA pieces");
// exception record: (first, packed); packed = extra index (9 bits) | extra count << 9
// (5 bits) | forward index << 14 (10 bits) | forward count << 24 (6 bits).
// extra record (one per earlier visit of a slot, in visit order): (token | row << 8,
// decay d of the visit, beta w of the visit)

// Chunk geometry: CC_ tokens per chunk, NW_ write rows and as many read rows
// per token.  Both configurations (16 x 32 and 8 x 64) have 512 write entries
// and 1024 staged rows per chunk, so the LDS budgets, the plan's size and the
// DMA pattern (32 DMAs of 32 rows of 32 bytes) are shared; only the index maps
// differ.  Rows of the fixed plan part are padded so that the apply kernel's
// LDS reads of them are free of bank conflicts.
template <int CC_, int NW_>
struct Geo {
    static constexpr int CC = CC_;         // tokens per chunk
    static constexpr int NW = NW_;         // write rows per token
    static constexpr int NR = NW_;         // read rows per token
    static constexpr int NQ = NW + NR;     // rows per token
    static constexpr int LOGNW = NW == 32 ? 5 : 6;
    static constexpr int RPD = 32 / CC;    // row indices q per DMA
    static constexpr int NMW = NW / 32;    // mask words per token
    static constexpr int OFFS_LD = 36, COEF_LD = NQ + 4, TB_LD = CC + 4;
    static constexpr int PL_OFFS = 0;                          // row byte offsets (see offs_word)
    static constexpr int PL_COEF = PL_OFFS + 32 * OFFS_LD;     // [t][q]: c (q < NW) or e (q >= NW)
    static constexpr int PL_TM = PL_COEF + CC * COEF_LD;       // [t][tau]: (I + A)^-1
    static constexpr int PL_BM = PL_TM + CC * TB_LD;           // [t][tau]
    static constexpr int PL_FIN = PL_BM + CC * TB_LD;          // [i][t][2]: decay d, beta w of write entry (t, i)
    static constexpr int PL_LAST = PL_FIN + NE * 2;            // [t][NMW] bit i: entry (t, i) is its slot's last visit
    static constexpr int PL_FIRST = PL_LAST + CC * NMW;        // [t][NMW] bit i: entry (t, i) is its slot's first visit
    static constexpr int PL_EXC = PL_FIRST + CC * NMW;         // [t][NMW] bit i: entry (t, i) has an exception record
    static constexpr int PL_EXCB = PL_EXC + CC * NMW;          // [t] index of token t's first exception record
    static constexpr int PL_HDR = PL_EXCB + CC;                // tail offsets of the extra pairs and forward rows
    static_assert(CC * NW == NE && CC * NQ == 2 * NE && 32 % CC == 0 && NW % 32 == 0, "chunk geometry");
    static_assert(PL_HDR + 4 <= PL_TAIL, "plan layout");
    static_assert(PL_COEF % 4 == 0 && COEF_LD % 4 == 0 && PL_TM % 4 == 0 && PL_BM % 4 == 0 &&
                      TB_LD % 4 == 0 && PL_FIN % 2 == 0 && PL_LAST % 2 == 0 && PL_HDR % 4 == 0,
                  "aligned vector reads of the plan");
    // row (q, t) is staged by DMA j = q / RPD of wave j % NWAVE, as row
    // (q % RPD) C + t of that DMA's 32; a lane's JW offsets for its wave are
    // contiguous
    static SSLP_DEVICE int offs_word(int q, int t) {
        const int j = q / RPD;
        return PL_OFFS + ((q % RPD) * CC + t) * OFFS_LD + (j % NWAVE) * JW + j / NWAVE;
    }
    static SSLP_DEVICE int coef_word(int t, int q) { return PL_COEF + t * COEF_LD + q; }
};
using GeoW32 = Geo<16, 32>;
using GeoW64 = Geo<8, 64>;

using namespace lds;  // the LDS / LDS-DMA helpers of the apply kernels

// Workgroup helpers of the plan kernels (256 threads, R elements each at
// positions p = tid + 256 r, r < R).

// Inclusive prefix sums of the 256 R values v[r] (position tid + 256 r): a
// scan inside each wavefront (lane shuffles), then the totals of the
// wavefronts before it from s_tot[4 R] behind one barrier.  s_tot must not be
// written again before every thread has passed a later barrier.
template <int R>
SSLP_DEVICE void block_scan(int (&v)[R], int* s_tot) {
    const int tid = (int)threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int o = __shfl_up(v[r], d, 64);
            v[r] += lane >= d ? o : 0;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int r = 0; r < R; ++r) s_tot[4 * r + w] = v[r];
    }
    __syncthreads();
    int before = 0;  // the totals of position blocks r' < r
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int mine = before, all = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int t = s_tot[4 * r + x];
            mine += x < w ? t : 0;
            all += t;
        }
        v[r] += mine;
        before += all;
    }
}

// One step (merge size KK, distance J) of the ascending bitonic sort of the
// 256 R keys k[r] at positions p = tid + 256 r: partners at distances up to
// 32 are exchanged inside the wavefront (xor_lane_c), at 256 and more inside
// the thread, at 64 and 128 through LDS (xbuf[] and key[] in turn, one
// barrier each: a buffer is rewritten only after a barrier that follows every
// read of it).
template <int R, int KK, int J>
SSLP_DEVICE void sort_step(uint64_t (&k)[R], uint64_t* key, uint64_t* xbuf, int& nx) {
    const int tid = (int)threadIdx.x;
    auto cx = [&](int r, uint64_t other) {
        const int p = tid + 256 * r;
        const bool keep_min = (((p & J) == 0) == ((p & KK) == 0));
        k[r] = ((k[r] < other) == keep_min) ? k[r] : other;
    };
    if constexpr (J >= 256) {
        constexpr int JR = J / 256;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if constexpr (JR < R) {
                if ((r & JR) == 0) {
                    const bool up = ((tid + 256 * r) & KK) == 0;
                    const uint64_t x = k[r], y = k[r | JR];
                    const uint64_t lo = x < y ? x : y, hi = x < y ? y : x;
                    k[r] = up ? lo : hi;
                    k[r | JR] = up ? hi : lo;
                }
            }
        }
    } else if constexpr (J >= 64) {
        uint64_t* buf = (nx++ & 1) ? xbuf : key;
#pragma unroll
        for (int r = 0; r < R; ++r) buf[tid + 256 * r] = k[r];
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) cx(r, buf[(tid + 256 * r) ^ J]);
    } else {
        const int lane = tid & 63;
#pragma unroll
        for (int r = 0; r < R; ++r) cx(r, xor_lane_c<J>(k[r], lane));
    }
}
template <int R, int KK, int J>
SSLP_DEVICE void sort_steps(uint64_t (&k)[R], uint64_t* key, uint64_t* xbuf, int& nx) {
    sort_step<R, KK, J>(k, key, xbuf, nx);
    if constexpr (J > 1) sort_steps<R, KK, J / 2>(k, key, xbuf, nx);
}
template <int R, int KK>
SSLP_DEVICE void sort_merges(uint64_t (&k)[R], uint64_t* key, uint64_t* xbuf, int& nx) {
    sort_steps<R, KK, KK / 2>(k, key, xbuf, nx);
    if constexpr (KK < 256 * R) sort_merges<R, KK * 2>(k, key, xbuf, nx);
}
// Ascending bitonic sort of the 256 R keys k[r] (position tid + 256 r), every
// stage resolved at compile time, left in key[] by position (the caller puts a
// barrier before reading it).  The LDS exchanges number 2 log2(R) + 3, an odd
// count starting on xbuf[], so the last one reads xbuf[] and key[] is free.
template <int R>
SSLP_DEVICE void block_sort_asc(uint64_t (&k)[R], uint64_t* key, uint64_t* xbuf) {
    static_assert(R == 2 || R == 4, "512 or 1024 keys");
    int nx = 1;
    sort_merges<R, 2>(k, key, xbuf, nx);
    // (key[] was last read in the exchange before the last one, which every
    // thread finished before the last one's barrier)
#pragma unroll
    for (int r = 0; r < R; ++r) key[(int)threadIdx.x + 256 * r] = k[r];
}

}  // namespace chunk
}  // namespace sslp
