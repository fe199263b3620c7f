// Records of the launcher stand-ins (launch_stubs.cpp).
#pragma once
#include "../../gated_deltanet_conv1d_amd/csrc/gdn_launch.hpp"

namespace stub {
struct Record {
  const char* which = nullptr;
  gdn::ConvFwdArgs conv_fwd{};
  gdn::ConvUpdateArgs conv_update{};
  gdn::GatingArgs gating{};
  gdn::StateCopyArgs state_copy{};
  gdn::RecurrentArgs recurrent{};
  gdn::DecodeArgs decode{};
  gdn::ChunkArgs chunk{};
  gdn::GemmaNormArgs norm{};
  gdn::ProjArgs proj{};
  gdn::SlotCheckArgs slot_check{};
};
extern Record last;               // the most recent launch (which == nullptr: none)
extern hipError_t next_result;    // what the next launches return
}  // namespace stub
