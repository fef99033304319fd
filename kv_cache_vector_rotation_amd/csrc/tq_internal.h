// Internal declarations shared by the host translation units of libturboquant.
#pragma once
#include <cstdint>

#include "turboquant.h"

namespace tq {

// Validates a layout: 3 <= d <= 256, 1 or 2 groups, each d_g >= 3 summing to d,
// m_g in [1, 4].
bool layout_valid(const tq_layout* l);

// Offsets of each group in channel / word units.
struct GroupGeom {
  int n_groups;
  int dim[2];
  int bits[2];
  int ch_off[2];        // first channel of the group in the rotated order
  int code_word_off[2]; // token-major: first code word of the group in a row
  int sign_word_off[2]; // token-major: first sign word of the group in a row
  int blk_code_off[2];  // block32: first code word of the group in a block
  int blk_sign_off[2];  // block32: first sign word of the group in a block
  int centroid_off[2];  // offset of the group's centroids in the concatenated array
  int boundary_off[2];  // offset of the group's boundaries
  tq_record_info info;
};

GroupGeom geometry(const tq_layout* l);

bool quantizer_pointers_valid(const tq_quantizer* q);

}  // namespace tq
