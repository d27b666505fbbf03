// sv_kernels.hpp -- gfx950 kernels of libspecverify.
//
// Pipeline of sv_verify_chain (one stream, no host synchronisation):
//   rowstats   streams the k target rows and k draft rows of every sequence
//              once; one wave64 per (row, tile) writes a softmax partial
//              (sum of exp2 against an integer reference) or, for rows at
//              temperature 0, the (max, lowest index) of the tile;
//   accept     one wave per sequence: combines the row partials, gathers the
//              2k logits at the draft tokens, forms tau_i in the log domain,
//              takes the first rejection with a ballot, writes the accepted
//              prefix and a descriptor of the final draw -- inside every
//              final_part workgroup for small draws, as its own kernel for
//              large ones, not at all without drafts;
//   final_part streams only the row(s) the final draw needs (target and draft
//              row a at a rejection, target row k after full acceptance) and
//              writes the statistics of every 64-vector segment: a residual's
//              terms are formed relative to themselves, with the sums that
//              correct log2(S_t / S_d) afterwards;
//   final_pick one wave per sequence: corrects a residual's masses, prefix
//              over the segment masses, picks the segment holding u * W and
//              rescans only that segment to find the token (the workgroup
//              forms the masses again when the correction cannot be trusted).
// When one wave can hold a sequence's 2k rows' partials and the draw fits one
// round of workgroups, rowstats and final_part run as one launch (fused):
// the drawing workgroups, after the streaming ones in the grid, read their
// sequence's partials as those are published, each tagged for the call, with
// no fence.  Small chains run in one workgroup per sequence (small), and
// plain sampling of many rows draws each row in one workgroup (row_draw).
// sv_verify_greedy and sv_verify_tree use argmax_rows (the streaming argmax)
// followed by a per-sequence finaliser; large calls stream in phases, a
// greedy chain's two phases in one launch (greedy_fused) and a tree's root
// rows with its first plan (tree_root_plan), handed over the same way.  sv_verify_tree_sampled streams the
// tree's rows (tree_rowstats), then walks every tree in rounds of launches
// (tree_round), with a one-workgroup walk (tree_sample) that finishes what
// the rounds leave.  sv_commit_tokens is one workgroup (commit_tokens).
//
// Scheme: "Accelerating Sonar through speculation" (Perplexity, 2025),
// sections "Speculative decoding", "Target-Draft" and "EAGLE"; acceptance
// and residual rule of Leviathan et al., first in that page's references;
// sampled trees: multi-step speculative sampling (SpecInfer, Miao et al.).
#pragma once

#include "sv_chain.hpp"
#include "sv_commit.hpp"
#include "sv_greedy_tree.hpp"
#include "sv_tiles.hpp"
#include "sv_tree_sampled.hpp"
