// vla_record.h -- layout of the per-chunk record that the penalty pass of the
// two-pass forward leaves in the workspace (16 tokens per chunk), read by the
// memory pass and by the scan form of the memory chain; and of the per-token
// record that the forward can leave for the gradient kernel.
#pragma once

namespace vla {
namespace rec {

constexpr int CH = 16;   // tokens per chunk

// One chunk's record (floats).  The memory pass copies records into LDS as
// they are, so the matrices it reads are laid out for that: a 16-column matrix
// X has X[i][c] at swz16(i, c >> 2) + (c & 3), a d-column one at
// swzd(i, c >> 2) + (c & 3).  The 16 x 16 factors are stored transposed (row i
// of the stored matrix is column i of the factor).
template <int D>
struct Rec {
    static constexpr int AH = 0;              // alpha^ [key][token]
    static constexpr int TT = D * CH;         // (I + N)^-1, transposed
    static constexpr int PT = TT + CH * CH;   // (Alpha^'Phi) o Up, transposed
    // even chunks c with a chunk c + 1: the key cross factor solved by the next
    // chunk's triangle, -(Alpha^_c' K^_{c+1}) (I + N_{c+1})^-1, and the readout
    // cross factor Alpha^_c' Phi_{c+1}, transposed (unset otherwise)
    static constexpr int QK = PT + CH * CH;
    static constexpr int QP = QK + CH * CH;
    static constexpr int RD = QP + CH * CH;   // 1 / den per token
    static constexpr int KH = RD + CH;        // k^ [token][key] (0 past T)
    static constexpr int PH = KH + CH * D;    // phi(q) [token][key]
    static constexpr int SIZE = PH + CH * D;  // a multiple of 4
};

// One token's record for the gradients (floats): z = A_{t-1} u^, alpha^, e, the
// key sum zkey_t (d each), then delta, 1/|y|, phi(q)'zkey_t, 1/|k|, 1/|u| and
// three unused floats.  Written by the two-pass forward when asked to (or by
// the gradient kernel's own per-token forward), read by its reverse sweep.
template <int D>
struct Keep {
    static constexpr int Z = 0, AL = D, E = 2 * D, ZK = 3 * D, SC = 4 * D;
    static constexpr int RS = 4 * D + 8;   // a multiple of 4
};

}  // namespace rec
}  // namespace vla
