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

}  // namespace chunk
}  // namespace sslp
