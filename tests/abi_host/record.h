// What the stub launchers of the host-only build saw: the last launch of
// each kind and how many launches there were.
#pragma once
#include "../../mixed_precision_tiled_amd/csrc/lamp_internal.h"

struct LaunchRecord {
  int n_quant = 0, n_quant_v = 0, n_mask = 0, n_template = 0, n_attn = 0, n_decode = 0;
  int n_exp8 = 0, n_scratch = 0;
  int attn_d = 0;
  lamp::QuantArgs quant{};
  lamp::VQuantArgs quant_v{};
  lamp::MaskArgs mask{};
  lamp::TemplateMaskArgs tmpl{};
  lamp::AttnArgs attn{};
  lamp::AttnConfig attn_cfg{};
  lamp::DecodeArgs decode{};
  int total() const {
    return n_quant + n_quant_v + n_mask + n_template + n_attn + n_decode + n_exp8;
  }
};

extern LaunchRecord g_rec;
extern char g_scratch[256];
