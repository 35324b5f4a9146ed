// vla_dpp_blocks.h -- inline-asm blocks of DPP multiply-adds used by the 16 x 16
// factorisations of the chunked kernel (vla_chunk_kernel.hip).
//
// Each block is one asm statement, so that no compiler-inserted instruction (a
// register copy, say) can land between the VALU write of a register and a later
// DPP read of it: gfx950 needs two wait states between the two, which the
// compiler does not track inside asm.  Every block starts with "s_nop 1" for the
// writes made before it, and inside a block consecutive self-updates of the same
// register are at least two instructions apart (s_nop fills the gap where fewer
// than three columns are in flight).
//
// v_fmac_f32_dpp d, s, m row_newbcast:L computes d += s[lane L of the 16-lane
// row] * m.
#pragma once

#define VLA_FSELF(X, M, L) \
    "v_fmac_f32_dpp %" #X ", %" #X ", %" #M " row_newbcast:" #L " row_mask:0xf bank_mask:0xf\n\t"

// Forward substitution with a unit lower triangular L, four columns at a time:
// operands %0..%3 = X[c] (column 4c + g of the inverse in lane group g, lane n =
// row n, starting as the unit vector), %4 + k = NL[k] = -L[n][k] (0 for n <= k).
// Step k (ascending) adds X[k] * NL[k] to every row; columns 4c + g with
// 4c > k still hold X[k] = 0 there and are skipped.
#define VLA_LINV_BLOCK \
    "s_nop 1\n\t" \
    VLA_FSELF(0, 4, 0) \
    "s_nop 1\n\t" \
    VLA_FSELF(0, 5, 1) \
    "s_nop 1\n\t" \
    VLA_FSELF(0, 6, 2) \
    "s_nop 1\n\t" \
    VLA_FSELF(0, 7, 3) \
    "s_nop 1\n\t" \
    VLA_FSELF(0, 8, 4) \
    VLA_FSELF(1, 8, 4) \
    "s_nop 0\n\t" \
    VLA_FSELF(0, 9, 5) \
    VLA_FSELF(1, 9, 5) \
    "s_nop 0\n\t" \
    VLA_FSELF(0, 10, 6) \
    VLA_FSELF(1, 10, 6) \
    "s_nop 0\n\t" \
    VLA_FSELF(0, 11, 7) \
    VLA_FSELF(1, 11, 7) \
    "s_nop 0\n\t" \
    VLA_FSELF(0, 12, 8) \
    VLA_FSELF(1, 12, 8) \
    VLA_FSELF(2, 12, 8) \
    VLA_FSELF(0, 13, 9) \
    VLA_FSELF(1, 13, 9) \
    VLA_FSELF(2, 13, 9) \
    VLA_FSELF(0, 14, 10) \
    VLA_FSELF(1, 14, 10) \
    VLA_FSELF(2, 14, 10) \
    VLA_FSELF(0, 15, 11) \
    VLA_FSELF(1, 15, 11) \
    VLA_FSELF(2, 15, 11) \
    VLA_FSELF(0, 16, 12) \
    VLA_FSELF(1, 16, 12) \
    VLA_FSELF(2, 16, 12) \
    VLA_FSELF(3, 16, 12) \
    VLA_FSELF(0, 17, 13) \
    VLA_FSELF(1, 17, 13) \
    VLA_FSELF(2, 17, 13) \
    VLA_FSELF(3, 17, 13) \
    VLA_FSELF(0, 18, 14) \
    VLA_FSELF(1, 18, 14) \
    VLA_FSELF(2, 18, 14) \
    VLA_FSELF(3, 18, 14)

// Back substitution with the unit upper triangular I + N, four columns at a
// time: operands %0..%3 = X[c] as above, %3 + k = NN[k] = -N[n][k] (0 for n >= k),
// k = 15 .. 1 (descending); columns 4c + g with 4c + 3 < k hold X[k] = 0 there
// and are skipped.
#define VLA_TINV_BLOCK \
    "s_nop 1\n\t" \
    VLA_FSELF(3, 18, 15) \
    "s_nop 1\n\t" \
    VLA_FSELF(3, 17, 14) \
    "s_nop 1\n\t" \
    VLA_FSELF(3, 16, 13) \
    "s_nop 1\n\t" \
    VLA_FSELF(3, 15, 12) \
    "s_nop 1\n\t" \
    VLA_FSELF(2, 14, 11) \
    VLA_FSELF(3, 14, 11) \
    "s_nop 0\n\t" \
    VLA_FSELF(2, 13, 10) \
    VLA_FSELF(3, 13, 10) \
    "s_nop 0\n\t" \
    VLA_FSELF(2, 12, 9) \
    VLA_FSELF(3, 12, 9) \
    "s_nop 0\n\t" \
    VLA_FSELF(2, 11, 8) \
    VLA_FSELF(3, 11, 8) \
    "s_nop 0\n\t" \
    VLA_FSELF(1, 10, 7) \
    VLA_FSELF(2, 10, 7) \
    VLA_FSELF(3, 10, 7) \
    VLA_FSELF(1, 9, 6) \
    VLA_FSELF(2, 9, 6) \
    VLA_FSELF(3, 9, 6) \
    VLA_FSELF(1, 8, 5) \
    VLA_FSELF(2, 8, 5) \
    VLA_FSELF(3, 8, 5) \
    VLA_FSELF(1, 7, 4) \
    VLA_FSELF(2, 7, 4) \
    VLA_FSELF(3, 7, 4) \
    VLA_FSELF(0, 6, 3) \
    VLA_FSELF(1, 6, 3) \
    VLA_FSELF(2, 6, 3) \
    VLA_FSELF(3, 6, 3) \
    VLA_FSELF(0, 5, 2) \
    VLA_FSELF(1, 5, 2) \
    VLA_FSELF(2, 5, 2) \
    VLA_FSELF(3, 5, 2) \
    VLA_FSELF(0, 4, 1) \
    VLA_FSELF(1, 4, 1) \
    VLA_FSELF(2, 4, 1) \
    VLA_FSELF(3, 4, 1)

// One column step of the LDL' factorisation (Crout order): for the CNT entries
// k = K0 .. K0+CNT-1,  acc += LD[k][lane J] * NL[k]  (LD[k] = L[.][k] d_k, NL[k]
// = -L[n][k]), CNT <= 8 so that the asm statement stays within 30 operands.
#define VLA_FBC(S, M) "v_fmac_f32_dpp %0, %" #S ", %" #M " row_newbcast:%[lane] row_mask:0xf bank_mask:0xf\n\t"
template <int J, int K0, int CNT>
__device__ __forceinline__ void ldl_block(float &acc, const float (&LD)[16], const float (&NL)[16])
{
    if constexpr (CNT == 1)
        asm volatile("s_nop 1\n\t" VLA_FBC(1, 2)
                     : "+v"(acc)
                     : "v"(LD[K0 + 0]), "v"(NL[K0 + 0]), [lane] "n"(J));
    else if constexpr (CNT == 2)
        asm volatile("s_nop 1\n\t" VLA_FBC(1, 3) VLA_FBC(2, 4)
                     : "+v"(acc)
                     : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), [lane] "n"(J));
    else if constexpr (CNT == 3)
        asm volatile("s_nop 1\n\t" VLA_FBC(1, 4) VLA_FBC(2, 5) VLA_FBC(3, 6)
                     : "+v"(acc)
                     : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), [lane] "n"(J));
    else if constexpr (CNT == 4)
        asm volatile("s_nop 1\n\t" VLA_FBC(1, 5) VLA_FBC(2, 6) VLA_FBC(3, 7) VLA_FBC(4, 8)
                     : "+v"(acc)
                     : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), [lane] "n"(J));
    else if constexpr (CNT == 5)
        asm volatile("s_nop 1\n\t" VLA_FBC(1, 6) VLA_FBC(2, 7) VLA_FBC(3, 8) VLA_FBC(4, 9) VLA_FBC(5, 10)
                     : "+v"(acc)
                     : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), [lane] "n"(J));
    else if constexpr (CNT == 6)
        asm volatile("s_nop 1\n\t" VLA_FBC(1, 7) VLA_FBC(2, 8) VLA_FBC(3, 9) VLA_FBC(4, 10) VLA_FBC(5, 11) VLA_FBC(6, 12)
                     : "+v"(acc)
                     : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), [lane] "n"(J));
    else if constexpr (CNT == 7)
        asm volatile("s_nop 1\n\t" VLA_FBC(1, 8) VLA_FBC(2, 9) VLA_FBC(3, 10) VLA_FBC(4, 11) VLA_FBC(5, 12) VLA_FBC(6, 13) VLA_FBC(7, 14)
                     : "+v"(acc)
                     : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), [lane] "n"(J));
    else if constexpr (CNT == 8)
        asm volatile("s_nop 1\n\t" VLA_FBC(1, 9) VLA_FBC(2, 10) VLA_FBC(3, 11) VLA_FBC(4, 12) VLA_FBC(5, 13) VLA_FBC(6, 14) VLA_FBC(7, 15) VLA_FBC(8, 16)
                     : "+v"(acc)
                     : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), [lane] "n"(J));
}

// Terms k = K0 .. K0+CNT-1 of LDL' column J (all with L[.][k] already known),
// alternating between two accumulators (k even -> a, odd -> b), so that they can
// be issued while the pivot of column J-1 is still being inverted; CNT <= 14.
#define VLA_FBC2(D, S, M) "v_fmac_f32_dpp %" #D ", %" #S ", %" #M " row_newbcast:%[lane] row_mask:0xf bank_mask:0xf\n\t"
template <int J, int K0, int CNT>
__device__ __forceinline__ void ldl_early(float &a, float &b, const float (&LD)[16], const float (&NL)[16])
{
    if constexpr (CNT == 1) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 3)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(NL[K0 + 0]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 3)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(NL[K0 + 0]), [lane] "n"(J));
    }
    else if constexpr (CNT == 2) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 4) VLA_FBC2(1, 3, 5)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 4) VLA_FBC2(0, 3, 5)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), [lane] "n"(J));
    }
    else if constexpr (CNT == 3) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 5) VLA_FBC2(1, 3, 6) VLA_FBC2(0, 4, 7)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 5) VLA_FBC2(0, 3, 6) VLA_FBC2(1, 4, 7)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), [lane] "n"(J));
    }
    else if constexpr (CNT == 4) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 6) VLA_FBC2(1, 3, 7) VLA_FBC2(0, 4, 8) VLA_FBC2(1, 5, 9)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 6) VLA_FBC2(0, 3, 7) VLA_FBC2(1, 4, 8) VLA_FBC2(0, 5, 9)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), [lane] "n"(J));
    }
    else if constexpr (CNT == 5) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 7) VLA_FBC2(1, 3, 8) VLA_FBC2(0, 4, 9) VLA_FBC2(1, 5, 10) VLA_FBC2(0, 6, 11)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 7) VLA_FBC2(0, 3, 8) VLA_FBC2(1, 4, 9) VLA_FBC2(0, 5, 10) VLA_FBC2(1, 6, 11)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), [lane] "n"(J));
    }
    else if constexpr (CNT == 6) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 8) VLA_FBC2(1, 3, 9) VLA_FBC2(0, 4, 10) VLA_FBC2(1, 5, 11) VLA_FBC2(0, 6, 12) VLA_FBC2(1, 7, 13)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 8) VLA_FBC2(0, 3, 9) VLA_FBC2(1, 4, 10) VLA_FBC2(0, 5, 11) VLA_FBC2(1, 6, 12) VLA_FBC2(0, 7, 13)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), [lane] "n"(J));
    }
    else if constexpr (CNT == 7) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 9) VLA_FBC2(1, 3, 10) VLA_FBC2(0, 4, 11) VLA_FBC2(1, 5, 12) VLA_FBC2(0, 6, 13) VLA_FBC2(1, 7, 14) VLA_FBC2(0, 8, 15)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 9) VLA_FBC2(0, 3, 10) VLA_FBC2(1, 4, 11) VLA_FBC2(0, 5, 12) VLA_FBC2(1, 6, 13) VLA_FBC2(0, 7, 14) VLA_FBC2(1, 8, 15)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), [lane] "n"(J));
    }
    else if constexpr (CNT == 8) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 10) VLA_FBC2(1, 3, 11) VLA_FBC2(0, 4, 12) VLA_FBC2(1, 5, 13) VLA_FBC2(0, 6, 14) VLA_FBC2(1, 7, 15) VLA_FBC2(0, 8, 16) VLA_FBC2(1, 9, 17)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 10) VLA_FBC2(0, 3, 11) VLA_FBC2(1, 4, 12) VLA_FBC2(0, 5, 13) VLA_FBC2(1, 6, 14) VLA_FBC2(0, 7, 15) VLA_FBC2(1, 8, 16) VLA_FBC2(0, 9, 17)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), [lane] "n"(J));
    }
    else if constexpr (CNT == 9) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 11) VLA_FBC2(1, 3, 12) VLA_FBC2(0, 4, 13) VLA_FBC2(1, 5, 14) VLA_FBC2(0, 6, 15) VLA_FBC2(1, 7, 16) VLA_FBC2(0, 8, 17) VLA_FBC2(1, 9, 18) VLA_FBC2(0, 10, 19)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 11) VLA_FBC2(0, 3, 12) VLA_FBC2(1, 4, 13) VLA_FBC2(0, 5, 14) VLA_FBC2(1, 6, 15) VLA_FBC2(0, 7, 16) VLA_FBC2(1, 8, 17) VLA_FBC2(0, 9, 18) VLA_FBC2(1, 10, 19)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), [lane] "n"(J));
    }
    else if constexpr (CNT == 10) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 12) VLA_FBC2(1, 3, 13) VLA_FBC2(0, 4, 14) VLA_FBC2(1, 5, 15) VLA_FBC2(0, 6, 16) VLA_FBC2(1, 7, 17) VLA_FBC2(0, 8, 18) VLA_FBC2(1, 9, 19) VLA_FBC2(0, 10, 20) VLA_FBC2(1, 11, 21)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(LD[K0 + 9]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), "v"(NL[K0 + 9]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 12) VLA_FBC2(0, 3, 13) VLA_FBC2(1, 4, 14) VLA_FBC2(0, 5, 15) VLA_FBC2(1, 6, 16) VLA_FBC2(0, 7, 17) VLA_FBC2(1, 8, 18) VLA_FBC2(0, 9, 19) VLA_FBC2(1, 10, 20) VLA_FBC2(0, 11, 21)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(LD[K0 + 9]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), "v"(NL[K0 + 9]), [lane] "n"(J));
    }
    else if constexpr (CNT == 11) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 13) VLA_FBC2(1, 3, 14) VLA_FBC2(0, 4, 15) VLA_FBC2(1, 5, 16) VLA_FBC2(0, 6, 17) VLA_FBC2(1, 7, 18) VLA_FBC2(0, 8, 19) VLA_FBC2(1, 9, 20) VLA_FBC2(0, 10, 21) VLA_FBC2(1, 11, 22) VLA_FBC2(0, 12, 23)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(LD[K0 + 9]), "v"(LD[K0 + 10]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), "v"(NL[K0 + 9]), "v"(NL[K0 + 10]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 13) VLA_FBC2(0, 3, 14) VLA_FBC2(1, 4, 15) VLA_FBC2(0, 5, 16) VLA_FBC2(1, 6, 17) VLA_FBC2(0, 7, 18) VLA_FBC2(1, 8, 19) VLA_FBC2(0, 9, 20) VLA_FBC2(1, 10, 21) VLA_FBC2(0, 11, 22) VLA_FBC2(1, 12, 23)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(LD[K0 + 9]), "v"(LD[K0 + 10]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), "v"(NL[K0 + 9]), "v"(NL[K0 + 10]), [lane] "n"(J));
    }
    else if constexpr (CNT == 12) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 14) VLA_FBC2(1, 3, 15) VLA_FBC2(0, 4, 16) VLA_FBC2(1, 5, 17) VLA_FBC2(0, 6, 18) VLA_FBC2(1, 7, 19) VLA_FBC2(0, 8, 20) VLA_FBC2(1, 9, 21) VLA_FBC2(0, 10, 22) VLA_FBC2(1, 11, 23) VLA_FBC2(0, 12, 24) VLA_FBC2(1, 13, 25)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(LD[K0 + 9]), "v"(LD[K0 + 10]), "v"(LD[K0 + 11]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), "v"(NL[K0 + 9]), "v"(NL[K0 + 10]), "v"(NL[K0 + 11]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 14) VLA_FBC2(0, 3, 15) VLA_FBC2(1, 4, 16) VLA_FBC2(0, 5, 17) VLA_FBC2(1, 6, 18) VLA_FBC2(0, 7, 19) VLA_FBC2(1, 8, 20) VLA_FBC2(0, 9, 21) VLA_FBC2(1, 10, 22) VLA_FBC2(0, 11, 23) VLA_FBC2(1, 12, 24) VLA_FBC2(0, 13, 25)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(LD[K0 + 9]), "v"(LD[K0 + 10]), "v"(LD[K0 + 11]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), "v"(NL[K0 + 9]), "v"(NL[K0 + 10]), "v"(NL[K0 + 11]), [lane] "n"(J));
    }
    else if constexpr (CNT == 13) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 15) VLA_FBC2(1, 3, 16) VLA_FBC2(0, 4, 17) VLA_FBC2(1, 5, 18) VLA_FBC2(0, 6, 19) VLA_FBC2(1, 7, 20) VLA_FBC2(0, 8, 21) VLA_FBC2(1, 9, 22) VLA_FBC2(0, 10, 23) VLA_FBC2(1, 11, 24) VLA_FBC2(0, 12, 25) VLA_FBC2(1, 13, 26) VLA_FBC2(0, 14, 27)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(LD[K0 + 9]), "v"(LD[K0 + 10]), "v"(LD[K0 + 11]), "v"(LD[K0 + 12]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), "v"(NL[K0 + 9]), "v"(NL[K0 + 10]), "v"(NL[K0 + 11]), "v"(NL[K0 + 12]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 15) VLA_FBC2(0, 3, 16) VLA_FBC2(1, 4, 17) VLA_FBC2(0, 5, 18) VLA_FBC2(1, 6, 19) VLA_FBC2(0, 7, 20) VLA_FBC2(1, 8, 21) VLA_FBC2(0, 9, 22) VLA_FBC2(1, 10, 23) VLA_FBC2(0, 11, 24) VLA_FBC2(1, 12, 25) VLA_FBC2(0, 13, 26) VLA_FBC2(1, 14, 27)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(LD[K0 + 9]), "v"(LD[K0 + 10]), "v"(LD[K0 + 11]), "v"(LD[K0 + 12]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), "v"(NL[K0 + 9]), "v"(NL[K0 + 10]), "v"(NL[K0 + 11]), "v"(NL[K0 + 12]), [lane] "n"(J));
    }
    else if constexpr (CNT == 14) {
        if constexpr (K0 % 2 == 0)
            asm volatile("s_nop 1\n\t" VLA_FBC2(0, 2, 16) VLA_FBC2(1, 3, 17) VLA_FBC2(0, 4, 18) VLA_FBC2(1, 5, 19) VLA_FBC2(0, 6, 20) VLA_FBC2(1, 7, 21) VLA_FBC2(0, 8, 22) VLA_FBC2(1, 9, 23) VLA_FBC2(0, 10, 24) VLA_FBC2(1, 11, 25) VLA_FBC2(0, 12, 26) VLA_FBC2(1, 13, 27) VLA_FBC2(0, 14, 28) VLA_FBC2(1, 15, 29)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(LD[K0 + 9]), "v"(LD[K0 + 10]), "v"(LD[K0 + 11]), "v"(LD[K0 + 12]), "v"(LD[K0 + 13]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), "v"(NL[K0 + 9]), "v"(NL[K0 + 10]), "v"(NL[K0 + 11]), "v"(NL[K0 + 12]), "v"(NL[K0 + 13]), [lane] "n"(J));
        else
            asm volatile("s_nop 1\n\t" VLA_FBC2(1, 2, 16) VLA_FBC2(0, 3, 17) VLA_FBC2(1, 4, 18) VLA_FBC2(0, 5, 19) VLA_FBC2(1, 6, 20) VLA_FBC2(0, 7, 21) VLA_FBC2(1, 8, 22) VLA_FBC2(0, 9, 23) VLA_FBC2(1, 10, 24) VLA_FBC2(0, 11, 25) VLA_FBC2(1, 12, 26) VLA_FBC2(0, 13, 27) VLA_FBC2(1, 14, 28) VLA_FBC2(0, 15, 29)
                         : "+v"(a), "+v"(b)
                         : "v"(LD[K0 + 0]), "v"(LD[K0 + 1]), "v"(LD[K0 + 2]), "v"(LD[K0 + 3]), "v"(LD[K0 + 4]), "v"(LD[K0 + 5]), "v"(LD[K0 + 6]), "v"(LD[K0 + 7]), "v"(LD[K0 + 8]), "v"(LD[K0 + 9]), "v"(LD[K0 + 10]), "v"(LD[K0 + 11]), "v"(LD[K0 + 12]), "v"(LD[K0 + 13]), "v"(NL[K0 + 0]), "v"(NL[K0 + 1]), "v"(NL[K0 + 2]), "v"(NL[K0 + 3]), "v"(NL[K0 + 4]), "v"(NL[K0 + 5]), "v"(NL[K0 + 6]), "v"(NL[K0 + 7]), "v"(NL[K0 + 8]), "v"(NL[K0 + 9]), "v"(NL[K0 + 10]), "v"(NL[K0 + 11]), "v"(NL[K0 + 12]), "v"(NL[K0 + 13]), [lane] "n"(J));
    }
}
