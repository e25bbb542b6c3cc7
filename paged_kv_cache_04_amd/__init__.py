"""GrowPage capacity-boundary event on MI355X (gfx950)."""
